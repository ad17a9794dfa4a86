// Merged dense weight W = deq(Wq) + A . B.
//
// "QLoRA (low-rank adapters on a quantized model)", "How it works", step 5:
// after training the adapters can be folded into the base weight; the result
// is a dense float matrix, off the quantization grid ("What the simulations
// show"), which qlora_quantize can take back to 4 bits at some loss.
//
// Per element, in fp32: w = L[code] * (q_b * s2_g), or L[code] * c_g in the
// 16-entry format (the two products the
// fused GEMMs form before their bf16 rounding), plus sum_j A[k][j] * B[j][n]
// in fp32, then one rounding to the output dtype.
//
// Two kernels.  For r % 8 == 0 (r = 0 included) the rank-r term is a dense
// contraction over r and runs on the matrix cores: merge_mfma_kernel starts
// each 32 x 32 MFMA accumulator from the dequantized fp32 weights and adds
// A.B in 16-rank steps, as 32 x 32 x 16 bf16 MFMAs for bf16 adapters (the
// products exact in fp32) or 32 x 32 x 2 fp32 MFMAs for fp32 adapters; the
// order of the fp32 additions is the hardware's.  The FMA kernel below
// serves the other ranks, summing in rank order.
//
// merge_mfma_kernel: 256 threads, a 64-row x 128-column tile; wavefront w owns
// rows 32 (w & 1) .. +31 and columns 64 (w >> 1) .. +63 as two 32 x 32 blocks.
// Each block is computed transposed, D = B^T-block . A^T-block + C, so that
// lane l holds W row l % 32 at columns 8 g + 4 (l / 32) + 0..3 (g = 0..3): the
// 16-B code vector of that row segment gives its nibbles, one block scale
// covers it, and A's 8 ranks per lane are contiguous (B's are 8 strided
// loads, L2-resident).  The tile then goes through a per-wave
// LDS buffer so that each store is a row-contiguous run (128 B of bf16, 256 B
// of fp32 per row), written with
// non-temporal stores (W is not read again by this launch).
//
// FMA kernel: 256 threads, a 64-row x 128-column tile of W.  Thread t owns rows
// 4 (t >> 4) .. +3 and columns 8 (t & 15) .. +7: four 4-byte code words (one
// 64-block each, so one scale per row) and a 4 x 8 fp32 accumulator of the
// rank-r term.  The rank runs in chunks of 32: the A chunk is staged
// transposed ([j][row], 68-float pitch) and the B chunk as is ([j][col]), so
// a thread reads one 16-B A quad and two 16-B B quads per rank index for 32
// multiply-adds.  The kernel is bound by HBM (the output write) for small r
// and by the fp32 multiply-adds (r per weight) as r grows.
#include "device.h"

namespace qlora {
namespace {

constexpr int kRows = 64, kCols = 128, kRC = 32, kAPitch = 68;

struct MergeArgs {
  const uint8_t *codes;
  const int8_t *q8;
  const float *s2;
  int64_t in, out;
  const void *A;      // [in x r]
  const void *B;      // [r x out]
  int r;
  void *W;            // [in x out]
  int g16;            // 16-entry format: s2 holds one fp32 scale per 16 weights
};

struct Levels {
  float L[16];
};

template <bool kAbf16>
__device__ __forceinline__ float load_adapter(const void *p, int64_t i) {
  if constexpr (kAbf16)
    return __uint_as_float(uint32_t(static_cast<const uint16_t *>(p)[i]) << 16);
  else
    return static_cast<const float *>(p)[i];
}

template <bool kAbf16, bool kWbf16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a, Levels lv) {
  __shared__ __align__(16) float sA[kRC][kAPitch];
  __shared__ __align__(16) float sB[kRC][kCols];
  __shared__ float sL[16];
  const int t = threadIdx.x, cg = t & 15, rg = t >> 4;
  const int64_t k0 = int64_t(blockIdx.y) * kRows, n0 = int64_t(blockIdx.x) * kCols;
  const int64_t ncols = min64(kCols, a.out - n0);          // 64 or 128
  if (t < 16) sL[t] = lv.L[t];

  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;

  for (int j0 = 0; j0 < a.r; j0 += kRC) {
    __syncthreads();                                       // previous chunk consumed
#pragma unroll
    for (int u = 0; u < kRows * kRC / 256; ++u) {          // A rows k0.., ranks j0..
      const int e = t + 256 * u, row = e / kRC, j = e % kRC;
      sA[j][row] = (j0 + j < a.r) ? load_adapter<kAbf16>(a.A, (k0 + row) * a.r + j0 + j) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kRC * kCols / 256; ++u) {          // B ranks j0.., columns n0..
      const int e = t + 256 * u, j = e / kCols, col = e % kCols;
      sB[j][col] = (j0 + j < a.r && col < ncols)
                       ? load_adapter<kAbf16>(a.B, int64_t(j0 + j) * a.out + n0 + col) : 0.0f;
    }
    __syncthreads();
    const int jn = a.r - j0 < kRC ? a.r - j0 : kRC;
    for (int j = 0; j < jn; ++j) {
      const f32x4_t av = *reinterpret_cast<const f32x4_t *>(&sA[j][4 * rg]);
      const f32x4_t b0 = *reinterpret_cast<const f32x4_t *>(&sB[j][8 * cg]);
      const f32x4_t b1 = *reinterpret_cast<const f32x4_t *>(&sB[j][8 * cg + 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][e] = __builtin_fmaf(av[i], b0[e], acc[i][e]);
          acc[i][4 + e] = __builtin_fmaf(av[i], b1[e], acc[i][4 + e]);
        }
      }
    }
  }
  __syncthreads();                                         // sL visible (r = 0 too)

  if (8 * cg >= ncols) return;
  const int64_t NB = a.out / 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = k0 + 4 * rg + i, col = n0 + 8 * cg;
    const int64_t flat = row * a.out + col;
    const uint32_t word = *reinterpret_cast<const uint32_t *>(a.codes + flat / 2);
    const int64_t blk = row * NB + col / 64;
    const float c = a.g16 ? a.s2[flat / 16] : float(a.q8[blk]) * a.s2[blk >> 8];
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = sL[(word >> (4 * e)) & 15u] * c + acc[i][e];
    if constexpr (kWbf16) {
      u32x4_t o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
      *reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(a.W) + flat) = o;
    } else {
      float *d = static_cast<float *>(a.W) + flat;
      *reinterpret_cast<f32x4_t *>(d) = f32x4_t{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4_t *>(d + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
    }
  }
}

// ---- matrix-core kernel ----
constexpr int kMRows = 64, kMCols = 128, kMBlocks = 2;    // blocks of 32 columns per wave

template <bool kAbf16, bool kWbf16, bool kG16>
__global__ __launch_bounds__(256) void merge_mfma_kernel(MergeArgs a, Levels lv) {
  constexpr int kES = kWbf16 ? 2 : 4;                      // output element bytes
  constexpr int kRowB = 32 * kMBlocks * kES;               // staged bytes per row
  constexpr int kPitch = kRowB + 16;
  __shared__ float sL[4][16];
  __shared__ __align__(16) uint8_t stage[4 * 32 * kPitch];
  const int t = threadIdx.x, w = t >> 6, l = t & 63, l32 = l & 31, h = l >> 5;
  const int64_t row0 = int64_t(blockIdx.y) * kMRows + 32 * (w & 1), row = row0 + l32;
  const int64_t nw0 = int64_t(blockIdx.x) * kMCols + (w >> 1) * (32 * kMBlocks);
  if (nw0 >= a.out) return;                                // whole wavefront; no block barrier
  const int nb = int(min64(kMBlocks, (a.out - nw0) / 32));
  const int64_t NB = a.out / 64;

  // Every load of the tile goes out first, with no condition around it (a
  // block past `nb` or a rank past r reads a valid element and is zeroed
  // or dropped), so a workgroup waits for memory once: the codes and scales
  // of columns n .. n + 31 (one block scale, or two 16-entry group scales)
  // and, for bf16 adapters, the operands of ranks 0..15.
  u32x4_t cw[kMBlocks];
  float sc[kMBlocks][2];
#pragma unroll
  for (int b = 0; b < kMBlocks; ++b) {
    const int64_t n = nw0 + 32 * (b < nb ? b : 0);
    cw[b] = *reinterpret_cast<const u32x4_t *>(a.codes + (row * a.out + n) / 2);
    if constexpr (kG16) {
      sc[b][0] = a.s2[(row * a.out + n) / 16];
      sc[b][1] = a.s2[(row * a.out + n) / 16 + 1];
    } else {
      const int64_t blk = row * NB + n / 64;
      sc[b][0] = float(a.q8[blk]) * a.s2[blk >> 8];
      sc[b][1] = sc[b][0];
    }
  }
  // bf16 adapters, ranks j0 .. j0 + 15: af = A[row][jh .. jh + 7] (jh = j0 +
  // 8 h), bf[b] = B[jh .. jh + 7][n] paired as the MFMA operand
  auto load_ab = [&](int j0, u32x4_t &af, u32x4_t (&bf)[kMBlocks]) {
    const uint16_t *A = static_cast<const uint16_t *>(a.A);
    const uint16_t *B = static_cast<const uint16_t *>(a.B);
    const int jh = j0 + 8 * h;
    const bool ok = jh < a.r;                               // r % 8 == 0: all 8 or none
    const u32x4_t av = *reinterpret_cast<const u32x4_t *>(A + row * a.r + (ok ? jh : 0));
    uint16_t raw[kMBlocks][8];
#pragma unroll
    for (int b = 0; b < kMBlocks; ++b) {
      const int64_t n = nw0 + 32 * (b < nb ? b : 0) + l32;
#pragma unroll
      for (int e = 0; e < 8; ++e) raw[b][e] = B[(ok ? jh + e : 0) * int64_t(a.out) + n];
    }
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    af = ok ? av : zero;
#pragma unroll
    for (int b = 0; b < kMBlocks; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bf[b][e] = ok ? uint32_t(raw[b][2 * e]) | (uint32_t(raw[b][2 * e + 1]) << 16) : 0u;
    }
  };
  u32x4_t af0 = {0u, 0u, 0u, 0u}, bf0[kMBlocks];
  if constexpr (kAbf16) {
    if (a.r > 0) load_ab(0, af0, bf0);
  }
  // the level table (read from the kernel arguments) after the tile's loads
  if (l < 16) sL[w][l] = lv.L[l];
  __builtin_amdgcn_wave_barrier();
  f32x16_t acc[kMBlocks];
#pragma unroll
  for (int b = 0; b < kMBlocks; ++b) {
#pragma unroll
    for (int i = 0; i < 16; ++i)                            // column 8 (i / 4) + 4 h + i % 4
      acc[b][i] = sL[w][(cw[b][i >> 2] >> (4 * (4 * h + (i & 3)))) & 15u] * sc[b][i >> 3];
  }
  if constexpr (kAbf16) {
  for (int j0 = 0; j0 < a.r; j0 += 16) {
    u32x4_t af = af0, bf[kMBlocks];
#pragma unroll
    for (int b = 0; b < kMBlocks; ++b) bf[b] = bf0[b];
    if (j0 > 0) load_ab(j0, af, bf);
#pragma unroll
    for (int b = 0; b < kMBlocks; ++b)
      if (b < nb) acc[b] = mfma32x32x16(bf[b], af, acc[b]);
  }
  } else {
  // fp32 adapters: 32 x 32 x 2 fp32 MFMAs, lane half h taking ranks
  // j0 + 8 h + s at step s (both operands alike, so each product pairs
  // A[k][j] with B[j][n]).
  const float *A = static_cast<const float *>(a.A);
  const float *B = static_cast<const float *>(a.B);
  for (int j0 = 0; j0 < a.r; j0 += 16) {
    const int jh = j0 + 8 * h;
    f32x4_t a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
    if (jh < a.r) {
      a0 = *reinterpret_cast<const f32x4_t *>(A + row * a.r + jh);
      a1 = *reinterpret_cast<const f32x4_t *>(A + row * a.r + jh + 4);
    }
#pragma unroll
    for (int b = 0; b < kMBlocks; ++b) {
      if (b < nb) {
        const int64_t n = nw0 + 32 * b + l32;
        float bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = jh < a.r ? B[int64_t(jh + e) * a.out + n] : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[e], e < 4 ? a0[e] : a1[e - 4], acc[b],
                                                        0, 0, 0);
      }
    }
  }
  }
  // Registers -> per-wave LDS rows -> row-contiguous stores.
#pragma unroll
  for (int b = 0; b < kMBlocks; ++b) {
    if (b < nb) {
      uint8_t *base = stage + (w * 32 + l32) * kPitch + 32 * kES * b;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint8_t *d = base + kES * (8 * g + 4 * h);
        if constexpr (kWbf16)
          *reinterpret_cast<u32x2_t *>(d) =
              u32x2_t{pack_bf16x2(acc[b][4 * g], acc[b][4 * g + 1]),
                      pack_bf16x2(acc[b][4 * g + 2], acc[b][4 * g + 3])};
        else
          *reinterpret_cast<f32x4_t *>(d) =
              f32x4_t{acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2], acc[b][4 * g + 3]};
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  constexpr int kLanesRow = kRowB / 16, kRowsPer = 64 / kLanesRow;
  const int pr = l / kLanesRow, pc = l % kLanesRow;
  if (pc < nb * (kLanesRow / kMBlocks)) {
    uint8_t *W = static_cast<uint8_t *>(a.W);
#pragma unroll
    for (int it = 0; it < 32 / kRowsPer; ++it) {
      const int rr = it * kRowsPer + pr;
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stage + (w * 32 + rr) * kPitch + 16 * pc);
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4_t *>(W + ((row0 + rr) * a.out + nw0) * kES + 16 * pc));
    }
  }
}

}  // namespace

hipError_t launch_merge(const uint8_t *codes, const int8_t *q8, const float *s2, int64_t in,
                        int64_t out, const void *A, const void *B, bool a_bf16, int32_t r,
                        void *W, bool w_bf16, int codebook, bool g16, hipStream_t s) {
  MergeArgs a{codes, q8, s2, in, out, A, B, int(r), W, g16 ? 1 : 0};
  Levels lv;
  const Tables &t = tables(codebook);
  for (int i = 0; i < 16; ++i) lv.L[i] = t.L[i];
  if (r % 8 == 0) {                                        // r = 0 included
    const dim3 mgrid(unsigned((out + kMCols - 1) / kMCols), unsigned(in / kMRows));
#define QLORA_MERGE(AB, WB)                                                                     \
  do {                                                                                          \
    if (g16) hipLaunchKernelGGL((merge_mfma_kernel<AB, WB, true>), mgrid, dim3(256), 0, s, a, lv);  \
    else hipLaunchKernelGGL((merge_mfma_kernel<AB, WB, false>), mgrid, dim3(256), 0, s, a, lv);     \
  } while (0)
    if (a_bf16) {
      if (w_bf16) QLORA_MERGE(true, true); else QLORA_MERGE(true, false);
    } else {
      if (w_bf16) QLORA_MERGE(false, true); else QLORA_MERGE(false, false);
    }
#undef QLORA_MERGE
    return hipGetLastError();
  }
  const dim3 grid(unsigned((out + kCols - 1) / kCols), unsigned(in / kRows));
  if (a_bf16) {
    if (w_bf16) hipLaunchKernelGGL((merge_kernel<true, true>), grid, dim3(256), 0, s, a, lv);
    else hipLaunchKernelGGL((merge_kernel<true, false>), grid, dim3(256), 0, s, a, lv);
  } else {
    if (w_bf16) hipLaunchKernelGGL((merge_kernel<false, true>), grid, dim3(256), 0, s, a, lv);
    else hipLaunchKernelGGL((merge_kernel<false, false>), grid, dim3(256), 0, s, a, lv);
  }
  return hipGetLastError();
}

}  // namespace qlora
