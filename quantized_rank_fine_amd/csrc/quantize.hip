// qlora_quantize kernel: blockwise absmax, fp32 nearest-level encode,
// nibble packing and int8 double quantization of the block scales.
//
// "LLMs · QLoRA", code listing: absmax per block of 64 consecutive weights,
// code = argmin_i |w/absmax - L_i|.  "QLoRA (low-rank adapters on a
// quantized model)", "What QLoRA adds": the block scales are quantized again
// to 8 bits (here: symmetric int8, one fp32 scale per 256 block scales).
//
// One workgroup (4 wavefronts) per double-quantization group of 256 blocks
// (64 KiB of fp32); wavefront w owns blocks 64 w .. 64 w + 63.  Load step j
// (0..7) covers 8 blocks: the 8 lanes of a block each take weights
// 4k .. 4k+3 and 32+4k .. 32+4k+3 (k = lane % 8), so each of the two load
// instructions of a step reads 8 whole 128-B lines, and the block absmax is an
// 8-lane DPP reduction.  All 16 loads are issued before the first is used;
// the buffer descriptors end at the last block, so a ragged last group loads
// zeros and drops its stores without a branch.
//
// The quotient x = w / c_b is the fp32 rounding of w * y in fp64, where
// y = 1/c_b is the fp64 reciprocal to within a few ulps (one per lane and
// block, see recip64).  That equals the IEEE fp32 quotient: the fp64 product
// is within 2^-50 (relative) of w / c_b, while a quotient of two fp32 numbers in
// the fp32 normal range is never an fp32 rounding midpoint and never within
// 2^-49 (relative) of one, so both round to the same fp32 value.  (Below the
// normal range x may differ, but every |x| < 2^-9 gets the same code.)
//
// Code lookup: code = #{j : x >= T_j} for the 15 exact fp32 decision
// thresholds.  The bucket of x is read off u = x + 3 in fp32 (u in [2, 4], so
// the top mantissa bits of u are a uniform grid of width 1/32 in x); the
// threshold gap (> 0.078) exceeds the bucket width, so a bucket holds at most
// one threshold and code = base + (x >= T_bucket), the compare on x itself.
// Rounding in x + 3 can move x at most 2^-23 up into the next bucket, which
// is harmless while no threshold lies that close below a bucket boundary (the
// nearest is 2^-10.7 away; the host checks this when it builds the table).
// The table {T_bucket, base} is built on the host and copied into LDS by
// each workgroup.
//
// The lab's 16-entry format ("QLoRA (low-rank adapters on a quantized
// model)", "The code, line by line": one scale per 16 consecutive entries, no
// double quantization) runs the same kernel with a 4-lane absmax: the 16
// weights 16q .. 16q + 15 of a block are elements 4k .. 4k + 3 (q = 0, 1) or
// 32 + 4k .. (q = 2, 3) of the four lanes k = 4 (q & 1) .. + 3, so each lane
// reduces its two halves over its quad, encodes each against its own group's
// absmax, and the quad's first lane stores the two fp32 group scales.
#include "device.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocksPerGroup = 256;
constexpr int kSteps = 8;                 // load steps per wavefront, 8 blocks each
constexpr int32_t kBufFlags = 0x00020000;
// Cache policy of the weight loads: non-temporal (streaming past the caches)
// for weights above 96 MiB, the default below.  Measured: at 4096 x 11008
// non-temporal loads take 37.7 us against 40.8 us with the default; at
// 4096 x 4096 the default takes 15.6 us against 16.9 us non-temporal.
constexpr int kNT = 2;
constexpr int64_t kNTBytes = int64_t(96) << 20;

__device__ __forceinline__ uint32_t bucket_of(float x) {
  return (__float_as_uint(x + 3.0f) >> 17) & uint32_t(kBuckets - 1);
}

__device__ __forceinline__ uint32_t code_of(float x, const BucketEntry *lut) {
  const BucketEntry e = lut[bucket_of(x)];
  return e.base + ((x >= e.T) ? 1u : 0u);
}

// y = 1/c in fp64 to within a few ulps: the hardware reciprocal refined by
// two Newton steps (y <- y + y (1 - c y), fused), a shorter dependent chain
// than the correctly rounded division.  The argument above needs the product
// w y within 2^-49 (relative) of w / c; with y a few fp64 ulps from 1/c it
// stays within 2^-50.  An infinite c gives y = 0, as the division would.
__device__ __forceinline__ double recip64(float c) {
  const double d = double(c);
  double y = __builtin_amdgcn_rcp(d);
  y = __builtin_fma(y, __builtin_fma(-d, y, 1.0), y);
  y = __builtin_fma(y, __builtin_fma(-d, y, 1.0), y);
  return __builtin_isinf(c) ? 0.0 : y;
}

// x = w / c as described above; y = 1/c in fp64 (y = 1 for a zero block, x = 0)
__device__ __forceinline__ uint32_t code4(f32x4_t w, double y, const BucketEntry *lut) {
  const uint32_t c0 = code_of(float(double(w.x) * y), lut);
  const uint32_t c1 = code_of(float(double(w.y) * y), lut);
  const uint32_t c2 = code_of(float(double(w.z) * y), lut);
  const uint32_t c3 = code_of(float(double(w.w) * y), lut);
  // element 2i -> low nibble of byte i, 2i+1 -> high nibble
  return c0 | (c1 << 4) | (c2 << 8) | (c3 << 12);
}

// max over the 8 lanes of a DPP half-row of non-negative fp32 bit patterns
// (0 is the identity, so each DPP move folds into its max)
__device__ __forceinline__ uint32_t row8_max(uint32_t m) {
  m = max(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0xB1, 0xF, 0xF, true)));   // quad [1,0,3,2]
  m = max(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0x4E, 0xF, 0xF, true)));   // quad [2,3,0,1]
  m = max(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0x141, 0xF, 0xF, true)));  // row_half_mirror
  return m;
}

// max over the 4 lanes of a DPP quad
__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  m = max(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0xB1, 0xF, 0xF, true)));   // quad [1,0,3,2]
  m = max(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0x4E, 0xF, 0xF, true)));   // quad [2,3,0,1]
  return m;
}

// max |w| over 4 weights (as absmax8)
__device__ __forceinline__ float absmax4(f32x4_t a) {
  float m;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|\n\t"
      "v_max_f32_e64 %0, %0, |%4|\n\t"
      "s_nop 1"                     // VALU write -> DPP read of the result
      : "=&v"(m)
      : "v"(a.x), "v"(a.y), "v"(a.z), "v"(a.w));
  return m;
}

// max |w| over the 8 weights of a lane (v_max3 with source modifiers; the
// library's fmaxf would first canonicalize every operand)
__device__ __forceinline__ float absmax8(f32x4_t a, f32x4_t b) {
  float m;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|\n\t"
      "v_max3_f32 %0, %0, |%4|, |%5|\n\t"
      "v_max3_f32 %0, %0, |%6|, |%7|\n\t"
      "v_max_f32_e64 %0, %0, |%8|\n\t"
      "s_nop 1"                     // VALU write -> DPP read of the result
      : "=&v"(m)
      : "v"(a.x), "v"(a.y), "v"(a.z), "v"(a.w), "v"(b.x), "v"(b.y), "v"(b.z), "v"(b.w));
  return m;
}

struct GroupRefs {
  __amdgpu_buffer_rsrc_t w, c;   // this group's weights and codes, ending at the last block
  __amdgpu_buffer_rsrc_t s;      // 16-entry format: its fp32 scales (4 per block)
  int nb;                        // blocks in this group
};

__device__ __forceinline__ GroupRefs group_refs(const float *W0, uint8_t *codes, float *scales,
                                                int64_t nblocks, int64_t g) {
  const int64_t rem = nblocks - g * kBlocksPerGroup;
  GroupRefs r;
  r.nb = rem < kBlocksPerGroup ? int(rem) : kBlocksPerGroup;
  r.w = __builtin_amdgcn_make_buffer_rsrc((void *)(W0 + g * kBlocksPerGroup * 64), (short)0,
                                          r.nb * 256, kBufFlags);
  r.c = __builtin_amdgcn_make_buffer_rsrc((void *)(codes + g * kBlocksPerGroup * 32), (short)0,
                                          r.nb * 32, kBufFlags);
  r.s = __builtin_amdgcn_make_buffer_rsrc((void *)(scales + g * kBlocksPerGroup * 4), (short)0,
                                          r.nb * 16, kBufFlags);
  return r;
}

template <int kAux>
__device__ __forceinline__ void load_group(__amdgpu_buffer_rsrc_t rW, uint32_t vw,
                                           f32x4_t (&v)[kSteps][2]) {
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    v[j][0] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rW, vw + j * 2048, 0, kAux));
    v[j][1] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rW, vw + j * 2048 + 128, 0, kAux));
  }
}

// codes of this wavefront's 64 blocks: block absmax to sc_blk, the 16-bit
// code groups to the wavefront's 2-KiB staging area, which then leaves in two
// 1-KiB contiguous stores
template <bool kG16>
__device__ __forceinline__ void encode_group(const f32x4_t (&v)[kSteps][2], const BucketEntry *lut,
                                             float *sc_blk, uint16_t *stage, int bl0,
                                             __amdgpu_buffer_rsrc_t rC, __amdgpu_buffer_rsrc_t rS) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, k = lane & 7;
  uint16_t *st = stage + (lane >> 3) * 16 + k;   // block bl0 - 64 wave, halfword k
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    const f32x4_t a = v[j][0], b = v[j][1];
    if constexpr (kG16) {
      // groups 16 q: q = k >> 2 (elements of a) and 2 + (k >> 2) (of b)
      const float ma = __uint_as_float(quad_max(__float_as_uint(absmax4(a))));
      const float mb = __uint_as_float(quad_max(__float_as_uint(absmax4(b))));
      const double ya = recip64(ma == 0.0f ? 1.0f : ma);
      const double yb = recip64(mb == 0.0f ? 1.0f : mb);
      st[j * 128] = uint16_t(code4(a, ya, lut));
      st[j * 128 + 8] = uint16_t(code4(b, yb, lut));
      if ((k & 3) == 0) {                        // one lane per quad stores its two scales
        const uint32_t off = uint32_t((bl0 + 8 * j) * 16 + (k >> 2) * 4);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ma), rS, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mb), rS, off + 8, 0, 0);
      }
    } else {
      const float m = __uint_as_float(row8_max(__float_as_uint(absmax8(a, b))));
      sc_blk[bl0 + 8 * j] = m;                  // the 8 lanes of the block agree
      const double y = recip64(m == 0.0f ? 1.0f : m);
      st[j * 128] = uint16_t(code4(a, y, lut));
      st[j * 128 + 8] = uint16_t(code4(b, y, lut));
    }
  }
  // LDS operations of one wavefront complete in order: the reads see all writes
  const u32x4_t *s4 = reinterpret_cast<const u32x4_t *>(stage);
  __builtin_amdgcn_raw_buffer_store_b128(s4[lane], rC, wave * 2048 + lane * 16, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(s4[64 + lane], rC, wave * 2048 + 1024 + lane * 16, 0, 0);
}

// double quantization of group g's 256 block scales (0 for padding blocks);
// sc_blk must be complete (barrier before)
__device__ __forceinline__ void double_quantize(const float *sc_blk, float *sred, int nb, int64_t g,
                                                int8_t *__restrict__ qscale,
                                                float *__restrict__ gscale) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float c = sc_blk[t];
  float gm = c;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
  if (lane == 0) sred[wave] = gm;
  __syncthreads();
  gm = fmaxf(fmaxf(sred[0], sred[1]), fmaxf(sred[2], sred[3]));
  const float s2 = gm / 127.0f;
  if (t < nb) {
    int q = 0;
    if (s2 != 0.0f) {
      q = (int)rintf(c / s2);
      q = q > 127 ? 127 : (q < -127 ? -127 : q);
    }
    qscale[g * kBlocksPerGroup + t] = (int8_t)q;
  }
  if (t == 0) gscale[g] = s2;
}

template <bool kG16, int kAux>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const float *__restrict__ W0, uint8_t *__restrict__ codes, int8_t *__restrict__ qscale,
    float *__restrict__ gscale, int64_t nblocks, QuantConsts qc) {
  __shared__ BucketEntry lut[kBuckets];
  __shared__ float sc_blk[kBlocksPerGroup];
  __shared__ float sred[kThreads / 64];
  __shared__ __attribute__((aligned(16))) uint16_t stage[kThreads / 64][1024];   // 2 KiB per wavefront

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int k = lane & 7;
  const int bl0 = wave * 64 + (lane >> 3);      // block (within the group) of step 0
  const uint32_t vw = uint32_t(bl0 * 256 + 16 * k);

  const int64_t g = blockIdx.x;
  const GroupRefs cur = group_refs(W0, codes, gscale, nblocks, g);
  BucketEntry own = {0.0f, 0u};
  if (t < kBuckets) own = qc.bucket[t];
  __builtin_amdgcn_sched_barrier(0);            // table read ahead of the weight loads
  f32x4_t v[kSteps][2];
  load_group<kAux>(cur.w, vw, v);
  if (t < kBuckets) lut[t] = own;
  __syncthreads();
  encode_group<kG16>(v, lut, sc_blk, stage[wave], bl0, cur.c, cur.s);
  if constexpr (!kG16) {
    __syncthreads();
    double_quantize(sc_blk, sred, cur.nb, g, qscale, gscale);
  }
}

}  // namespace

hipError_t launch_quantize(const float *W0, uint8_t *codes, int8_t *qscale, float *gscale,
                           int64_t nblocks, int codebook, bool g16, hipStream_t s) {
  const int64_t groups = (nblocks + kBlocksPerGroup - 1) / kBlocksPerGroup;
  if (groups == 0) return hipSuccess;
  const Tables &t = tables(codebook);
  if (!t.quant.ok) return hipErrorInvalidValue;
  const dim3 grid = dim3(unsigned(groups));
  const bool nt = nblocks * 256 > kNTBytes;
#define QLORA_Q(G, AUX)                                                                      \
  hipLaunchKernelGGL((quantize_kernel<G, AUX>), grid, dim3(kThreads), 0, s, W0, codes, qscale, \
                     gscale, nblocks, t.quant)
  if (g16) {
    if (nt) QLORA_Q(true, kNT); else QLORA_Q(true, 0);
  } else {
    if (nt) QLORA_Q(false, kNT); else QLORA_Q(false, 0);
  }
#undef QLORA_Q
  return hipGetLastError();
}

}  // namespace qlora
