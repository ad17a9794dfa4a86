// Fused dequantizing GEMMs of the adapted linear layer on bf16 matrix cores.
//
//   forward  y  = X . deq(Wq) + XA . B          (contraction over `in`)
//   backward dX = dY . deq(Wq)^T + G . A^T      (contraction over `out`)
//
// "QLoRA (low-rank adapters on a quantized model)", "What QLoRA adds": the
// frozen 4-bit weights are expanded to bf16 on the fly for each matmul and
// never updated; "How it works": W = Wq + A B, the rank-r term being "one
// small extra matmul" -- here it runs on the same accumulators after the
// main K loop.
//
// Workgroup: 256 threads = 4 wavefronts; tile 256 (M) x 128 (N) x 64 (K).
// Wavefront w owns columns 64 (w & 1) .. +63 and half of every K tile
// (k half w >> 1), as 8 x 2 tiles of v_mfma_f32_32x32x16_bf16; every weight of
// the tile is expanded exactly once per workgroup and every activation
// fragment read from LDS feeds two MFMAs.  The two k halves are summed in the
// epilogue.  Tiles stream through a 4-stage LDS ring filled by
// buffer_load ... lds (the K offset is a scalar; rows past M read as 0).
// Activation tiles are row-major (128 B per row) with the 16-B chunks of a row
// XOR-swizzled by (row >> 1) & 7: the 16 rows one MFMA fragment read touches
// per 16-lane group then fall on 16 distinct 16-B bank groups of the 256-B
// LDS bank window.  The weight tile is raw packed codes (1/4 of its bf16
// size) and the per-block scales c_b = q_b * s2_g come from a small fp32
// array laid out [block][row].
// K slots are permuted inside each 64-wide K tile: lane half h (lanes 32h..)
// of the MFMA owns k = 32h .. 32h+31 (8 per substep), for both operands.
//
// Forward: the code tile is 64 k-rows x 128 n-cols, n-contiguous, and the
// scale of a weight depends on its k row (and the wavefront's block column).
// A lane reads 8 bytes of one k row (16 consecutive columns, one scale),
// expands them through that row's per-scale table and writes the bf16 values
// to a per-wavefront LDS scratch, which is read back transposed with
// ds_read_b64_tr_b16 as the MFMA B fragments.
// Backward dX: the code tile is 128 W-rows x 64 W-cols and the contraction
// runs along a W row: one 8-byte read gives a lane the 16 consecutive k of
// its k half, all under one scale (the K tile is one 64-wide block).
//
// Expansion: w = bf16(L[code] * scale), the fp32 product rounded once.  For
// each scale a per-scale table holds the 8 magnitudes bf16(|L|_m * scale) as
// two v_perm byte planes (the level set is sign-symmetric), so a code becomes
// its bf16 weight by table lookup and a sign bit.
//
// The dX GEMM can also form dB = XA^T . dY from the dY tiles it streams (see
// DbFold below), so that the backward reads dY once.
#include <type_traits>

#include "device.h"

namespace qlora {
namespace {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kStages = 4;
constexpr int kXBytes = BM * BK * 2;     // 32 KiB activation tile
constexpr int kCBytes = 4096;            // code tile
constexpr uint32_t kBufFlags = 0x00020000u;

// LDS geometry per scale format.  64-weight blocks (kG16 = false): one fp32
// scale per (64-column block, row) -- 512 B of a 1-KiB slot per stage; the
// forward's per-wavefront expansion scratch holds 16 k rows x 64 columns of
// bf16 with a 176-B (44-dword) row pitch: the expansion's 16-B writes hit
// every LDS bank exactly 4 times per instruction (the minimum) and the
// transposed reads at most 3 times (minimum 2).  16-entry groups (kG16 =
// true): one fp32 scale per (16-column group, row) -- 2 KiB per stage, paid
// for with an unpadded scratch pitch, so the workgroup takes all 160 KiB.
template <bool kG16>
struct Geo {
  static constexpr int kSBytes = kG16 ? 2048 : 1024;
  static constexpr int kStageBytes = kXBytes + kCBytes + kSBytes;
  static constexpr int kRingBytes = kStages * kStageBytes;
  static constexpr int kXPitch = kG16 ? 64 : 88;                 // elements
  static constexpr int kScratchBytes = 16 * kXPitch * 2;        // per wavefront
  static constexpr int kLdsBytes = kRingBytes + 4 * kScratchBytes;
  // loads per wavefront and tile: 8 X + 1 code + the scale loads
  static constexpr int kLoadsPerTile = kG16 ? 11 : 10;
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
};

__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0) over [base, base + bytes); loads past the
// end return zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : int32_t(bytes));
  rsrc_t r = {int32_t(uint32_t(b)), int32_t(uint32_t(b >> 32) & 0xffffu), n, int32_t(kBufFlags)};
  r[0] = __builtin_amdgcn_readfirstlane(r[0]);
  r[1] = __builtin_amdgcn_readfirstlane(r[1]);
  r[2] = __builtin_amdgcn_readfirstlane(r[2]);
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_char *)(p)));
}

// buffer_load ... lds: each lane's 16 (or 4) bytes land at M0 + 16*lane (4*lane).
// Issued from inline assembly so that the compiler does not fold its own
// conservative wait for these LDS writes into the pipeline's vmcnt waits; the
// ring protocol below waits and synchronizes explicitly.  No register is
// written by these loads.
// The LDS address and the scalar offset are wavefront-uniform by construction;
// readfirstlane keeps them in SGPRs wherever the compiler cannot prove it.
__device__ __forceinline__ void lds_load16(rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

// ------------------------------------------------------------- expansion
// Per-scale level table for a uniform scale s: the 8 magnitudes
// bf16(|L|_m * s) (fp32 product, one rounding) as two v_perm byte planes --
// lo[w] holds the low bytes of m = 4w..4w+3, hi[w] the high bytes.  A weight
// with code c is then +-table[m] (sign-symmetric levels), bit-identical to
// bf16(L[c] * s).
struct ScaledTable {
  uint32_t lo[2], hi[2];
};

__device__ __forceinline__ ScaledTable scaled_table(float s, const ExpandConsts &t) {
  uint32_t p[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) p[q] = pack_bf16x2(t.mag[2 * q] * s, t.mag[2 * q + 1] * s);
  ScaledTable r;
  r.lo[0] = perm_b32(p[1], p[0], 0x06040200u);
  r.lo[1] = perm_b32(p[3], p[2], 0x06040200u);
  r.hi[0] = perm_b32(p[1], p[0], 0x07050301u);
  r.hi[1] = perm_b32(p[3], p[2], 0x07050301u);
  return r;
}

// 8 codes (nibble t of d = k slot t) -> the bf16x8 MFMA operand (k pairs).
__device__ __forceinline__ u32x4_t expand8_table(uint32_t d, const ScaledTable &T) {
  // magnitude index m = c - 8 (c >= 8) or 7 - c (c < 8), per byte; nt has
  // 0x08 in the bytes of negative levels
  const uint32_t nl = ~d & 0x08080808u;                     // even k slots
  const uint32_t ml = (d ^ (nl - (nl >> 3))) & 0x07070707u;
  const uint32_t dh = d >> 4;                               // odd k slots
  const uint32_t nh = ~dh & 0x08080808u;
  const uint32_t mh = (dh ^ (nh - (nh >> 3))) & 0x07070707u;
  const uint32_t LL = perm_b32(T.lo[1], T.lo[0], ml);       // low bytes, k = 0,2,4,6
  const uint32_t HL = perm_b32(T.hi[1], T.hi[0], ml) | (nl << 4);
  const uint32_t LH = perm_b32(T.lo[1], T.lo[0], mh);       // k = 1,3,5,7
  const uint32_t HH = perm_b32(T.hi[1], T.hi[0], mh) | (nh << 4);
  const uint32_t A0 = perm_b32(HL, LL, 0x05010400u);        // bf16 k0, k2
  const uint32_t B0 = perm_b32(HH, LH, 0x05010400u);        // bf16 k1, k3
  const uint32_t A1 = perm_b32(HL, LL, 0x07030602u);        // k4, k6
  const uint32_t B1 = perm_b32(HH, LH, 0x07030602u);        // k5, k7
  u32x4_t r;
  r[0] = perm_b32(B0, A0, 0x05040100u);
  r[1] = perm_b32(B0, A0, 0x07060302u);
  r[2] = perm_b32(B1, A1, 0x05040100u);
  r[3] = perm_b32(B1, A1, 0x07060302u);
  return r;
}

// Transposed read of a row-major bf16 LDS tile T (pitch kXPitch): lane l
// receives column cb + (l & 31), rows 8 (l >> 5) .. +7 -- one lane of a
// v_mfma_f32_32x32x16 B operand -- from two ds_read_b64_tr_b16 (each: 16
// lanes x 4 rows -> 4 columns).
template <int kXPitch>
__device__ __forceinline__ u32x4_t lds_col8_32(const char *T, int cb) {
  const int lane = threadIdx.x & 63, g = lane >> 4, i16 = lane & 15;
  const int q = i16 & 3, tq = i16 >> 2;
  const int rr = 8 * (g >> 1) + tq;
  const int col = cb + 16 * (g & 1) + 4 * q;
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  lds_char *base = (lds_char *)(T);
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + (rr * kXPitch + col) * 2));
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + ((rr + 4) * kXPitch + col) * 2));
  const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
}

// Scheduling hint for one half-step: 16 MFMAs, each followed by one LDS read
// (for the first kNDS) and kNV VALU instructions.
template <int kNDS, int kNV>
__device__ __forceinline__ void sched_pattern() {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
    if (q < kNDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
    __builtin_amdgcn_sched_group_barrier(0x002, kNV, 0);                  // VALU
  }
}

// Map the linear workgroup id to a (m-tile, n-tile).  Workgroups are dealt
// to the 8 XCDs round-robin; T = (id % 8) * (n / 8) + id / 8 gives each XCD a
// contiguous run of tiles, which share m-tiles (their activation rows stay in
// that XCD's L2).
__device__ __forceinline__ void tile_of(int nt_count, int &mt, int &nt) {
  const int n = gridDim.x, id = blockIdx.x;
  const int T = (n % 8 == 0) ? (id % 8) * (n / 8) + id / 8 : id;
  mt = T / nt_count;
  nt = T % nt_count;
}

// LDS address (bytes) of the 16-B chunk `c` of activation row `row`.
__device__ __forceinline__ uint32_t xoff(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }


// ------------------------------------------------------- shared main loop
//
// Wavefront roles: column half ch = wave & 1 owns 64 columns of the tile (two
// 32-wide MFMA column blocks b), and k half kh = wave >> 1 owns two of the
// four k16 substeps of every K tile (u = 2 kh + j, j = 0, 1).  Each wavefront
// therefore accumulates a 256 x 64 partial over half of K (acc[b][i]); the two
// k halves are summed once, after the loop.  Per K tile a wavefront reads 16
// activation fragments from LDS and expands 4 weight fragments for 32 MFMAs.
//
// The loop is software-pipelined by one substep: while the MFMAs of substep j
// run, the operands of the next substep are read and expanded.  The workgroup
// barrier sits between the two substeps of a tile, so the operands of the
// next tile are prepared while the second substep's MFMAs run.
//
// kFwd selects the weight-tile layout and expansion; everything else is
// common.  Arguments:
//   A16: activations bf16 [M x K]; codes; cs: scales fp32 [blocks][rows].
//   Forward: weight rows = K (k), columns = N; cs row count = K.
//   dX:      weight rows = N (i), columns = K; cs row count = N.
// dB = XA^T . dY taken over by the dX GEMM (ranks r <= 16).  The workgroup of
// token block tb = m0 / 256 and output-column block cw = n0 / 128 multiplies
// the dY tiles kt = cw, cw + ncw, ... of its LDS ring by XA^T over its 256
// tokens: wavefront w owns the 16 dB columns 64 kt + 16 w .. + 15, eight
// v_mfma_f32_16x16x32_bf16 with XA^T (rows = ranks) as the A operand, held in
// registers from the start, and dY read transposed out of the swizzled tile
// with ds_read_b64_tr_b16.  Every column of dB is formed once per token block,
// as part[tb][n][j] (fp32), which a fixed-order reduction sums over tb.
struct DbFold {
  const uint16_t *xat;   // XA^T bf16 [16 x ldm], zero for ranks >= r, tokens >= M
  int64_t ldm;
  float *part;           // [ceil(M / 256)][K][r]; nullptr: no dB here
  int r;
  int ncw;               // output-column blocks of the launch
};
constexpr int kMaxDbTiles = 4;               // dB tiles per workgroup, at most
constexpr uint32_t kNoStore = 0xffffffffu;   // no dB results for this lane

// 4 consecutive rows of one column of a bf16 tile, transposed across a
// 16-lane group (see lds_col8_32).
__device__ __forceinline__ u32x2_t lds_tr4(const char *p) {
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)((lds_char *)(p)));
  return __builtin_bit_cast(u32x2_t, v);
}

// The eight dB products of one tile as one chain on VGPR accumulators.  Every
// AGPR holds a GEMM accumulator, and the builtin form would take four of them
// (the compiler then moves an accumulator block through VGPRs on every
// iteration).  The products accumulate back to back on the same registers
// (srcC = vdst, the form the hardware forwards); the leading s_nop covers a
// VALU write of an operand just before, the trailing ones the wait states
// before any VALU or memory instruction reads the result.
__device__ __forceinline__ f32x4_t db_chain(const u32x4_t (&a)[8], const u32x4_t (&b)[8]) {
  f32x4_t d = {0.f, 0.f, 0.f, 0.f};
  asm volatile(
      "s_nop 4\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %1, %9, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %10, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %11, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %12, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %13, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %14, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %7, %15, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %8, %16, %0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(d)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]), "v"(b[6]), "v"(b[7]));
  return d;
}

template <bool kFwd, bool kG16>
__device__ __forceinline__ void gemm_mainloop(const uint16_t *__restrict__ A16, int64_t M, int64_t K,
                                              int64_t N, const uint8_t *__restrict__ codes,
                                              const float *__restrict__ cs, int64_t m0, int64_t n0,
                                              const ExpandConsts &tb, char *smem,
                                              f32x16_t (&acc)[2][8], const DbFold &dbf) {
  using G = Geo<kG16>;
  constexpr int kStageBytes = G::kStageBytes, kRingBytes = G::kRingBytes;
  constexpr int kXPitch = G::kXPitch, kScratchBytes = G::kScratchBytes;
  constexpr int kLoadsPerTile = G::kLoadsPerTile;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: LDS targets go to M0
  const int ch = wave & 1, kh = wave >> 1;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int KT = int(K / BK);

  // ---- buffer descriptors (per workgroup) and per-lane constant offsets
  const rsrc_t rX = make_rsrc(A16 + m0 * K, (M - m0) * K * 2);
  uint32_t vx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (8 * wave + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    vx[j] = uint32_t(row) * uint32_t(K) * 2u + uint32_t(c) * 16u;
  }
  rsrc_t rC, rS;
  uint32_t vc, vs, vs2 = 0;
  {
    const int s = 64 * wave + lane;               // 16-B slot of the code tile
    if constexpr (kFwd) {
      // 64 k-rows x 4 pieces; slot s -> row 8*(s>>5) + (s&7), piece (s>>3)&3
      const int row = 8 * (s >> 5) + (s & 7);
      int q = (s >> 3) & 3;
      // A ragged last tile (N % 128 == 64) has only pieces 0 and 1 inside the
      // row; pieces 2 and 3 re-read them (their columns are never stored).
      // The range check of a raw buffer covers the per-lane offset only, so
      // every address must stay inside the row by construction.
      if (n0 / 2 + 16 * q + 16 > N / 2) q -= 2;
      rC = make_rsrc(codes + n0 / 2, K * (N / 2) - n0 / 2);
      vc = uint32_t(row) * uint32_t(N / 2) + 16u * q;
      if constexpr (kG16) {
        // scales as stored, [k][N/16]: wavefront w gathers groups gg = 2 w
        // and 2 w + 1 of the tile's eight (lane = k row; a group past N,
        // in a ragged last tile, reads the last group: never stored)
        const int64_t ng = N / 16;
        rS = make_rsrc(cs, K * ng * 4);
        const int64_t g0 = n0 / 16 + 2 * wave;
        vs = uint32_t(int64_t(lane) * ng + (g0 < ng ? g0 : ng - 1)) * 4u;
        vs2 = uint32_t(int64_t(lane) * ng + (g0 + 1 < ng ? g0 + 1 : ng - 1)) * 4u;
      } else {
        // scales: block column nb0 + (wave & 1), 64 k per tile
        const int64_t nb = n0 / 64 + (wave & 1);
        rS = make_rsrc(cs, (N / 64) * K * 4);
        vs = uint32_t(nb * K + lane) * 4u;
      }
    } else {
      // 128 W-rows x 2 pieces; slot s -> row 8*(s>>4) + (s&7), piece (s>>3)&1
      const int row = 8 * (s >> 4) + (s & 7), q = (s >> 3) & 1;
      rC = make_rsrc(codes + n0 * (K / 2), (N - n0) * (K / 2));
      vc = uint32_t(row) * uint32_t(K / 2) + 16u * q;
      if constexpr (kG16) {
        // scales as stored, [W row][K/16]: wavefront w gathers group w of the
        // tile's four for W rows 0..63 and 64..127 (rows past N clamped)
        const int64_t ng = K / 16;
        rS = make_rsrc(cs, N * ng * 4);
        const int64_t r0 = n0 + lane, r1 = n0 + 64 + lane;
        vs = uint32_t((r0 < N ? r0 : N - 1) * ng + wave) * 4u;
        vs2 = uint32_t((r1 < N ? r1 : N - 1) * ng + wave) * 4u;
      } else {
        rS = make_rsrc(cs, (K / 64) * N * 4);
        // the K offset is scalar (outside the range check): clamp the row
        const int64_t srow = n0 + 64 * (wave & 1) + lane;
        vs = uint32_t(srow < N ? srow : N - 1) * 4u;
      }
    }
  }

  const uint32_t lds0 = lds_addr(smem);
  // Range checks of these raw buffers apply to the per-lane offset only; the
  // scalar K offset never moves an address out of its row (or array).
  auto issue = [&](int kt, int stage) {
    const uint32_t base = lds0 + uint32_t(stage * kStageBytes);
    const uint32_t sx = uint32_t(kt) * BK * 2u;
#pragma unroll
    for (int j = 0; j < 8; ++j) lds_load16(rX, base + (8 * wave + j) * 1024, vx[j], sx);
    uint32_t sc, ss;
    if constexpr (kFwd) {
      sc = uint32_t(kt) * BK * uint32_t(N / 2);
      ss = kG16 ? uint32_t(kt) * BK * uint32_t(N / 16) * 4u : uint32_t(kt) * BK * 4u;
    } else {
      sc = uint32_t(kt) * (BK / 2);
      ss = kG16 ? uint32_t(kt) * (BK / 16) * 4u : uint32_t(kt) * uint32_t(N) * 4u;
    }
    lds_load16(rC, base + kXBytes + wave * 1024, vc, sc);
    if constexpr (kG16) {
      lds_load4(rS, base + kXBytes + kCBytes + (2 * wave) * 256, vs, ss);
      lds_load4(rS, base + kXBytes + kCBytes + (2 * wave + 1) * 256, vs2, ss);
    } else {
      lds_load4(rS, base + kXBytes + kCBytes + wave * 256, vs, ss);
    }
  };

  // ---- per-lane LDS read offsets inside a stage
  // activation fragment (i, j): row 32 i + l32, 16-B chunk 4 h2 + 2 kh + j
  uint32_t xo[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) xo[j] = xoff(l32, 4 * h2 + 2 * kh + j);   // + 32 i rows = 4096 i B
  uint32_t co[2];                   // code read offset per column block b (dX) or substep j (fwd)
  // Forward expansion layout: lane (er = lane >> 2, seg = lane & 3) expands
  // 16 consecutive columns 16 seg .. of the wavefront's 64 for k row
  // kr(j) = 32 (er >> 3) + 8 (2 kh + j) + (er & 7) of substep j; scratch row
  // er, so that scratch rows 8 h2 .. 8 h2 + 7 are the k slots of lane half h2.
  const int er = lane >> 2, seg = lane & 3;
  uint32_t sco = 0;                 // fwd: scale offset (floats) of k row kr(0)
  if constexpr (kFwd) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kr = 32 * (er >> 3) + 8 * (2 * kh + j) + (er & 7);
      const int piece = 2 * ch + (seg >> 1);
      co[j] = uint32_t(((kr >> 3) * 32 + piece * 8 + (kr & 7)) * 16 + 8 * (seg & 1));
    }
    sco = uint32_t(ch * 64 + 32 * (er >> 3) + 16 * kh + (er & 7));
  } else {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int row = 64 * ch + 32 * (b ^ kh) + l32;        // accumulator b = column block b ^ kh
      co[b] = uint32_t(((row >> 3) * 16 + h2 * 8 + (row & 7)) * 16 + 8 * kh);
    }
  }
  // scale read offset (bytes into the scale area of a stage).  16-entry
  // groups: forward [group gg][k], the lane's 16 columns being group 4 ch +
  // seg; dX [group gg][W row], the lane's k run (8 (2 kh + j) + 32 h2 ..
  // + 7, both substeps) lying in group 2 h2 + kh.
  uint32_t so;
  if constexpr (kG16) {
    const int kr0 = 32 * (er >> 3) + 16 * kh + (er & 7);      // k row kr(0)
    so = kFwd ? uint32_t(((4 * ch + seg) * 64 + kr0) * 4)
              : uint32_t(((2 * h2 + kh) * 128 + ch * 64 + l32) * 4);
  } else {
    so = kFwd ? sco * 4u : uint32_t((ch * 64 + l32) * 4);
  }
  char *scr = smem + kRingBytes + wave * kScratchBytes;              // fwd expansion scratch
  const uint32_t swo = uint32_t((er * kXPitch + 16 * seg) * 2);      // this lane's scratch bytes

  // Per tile and lane: nib[b][j] = 8 codes (k slots 32 h2 + 8 (2 kh + j) +
  // 0..7) of column block b; sc = the scales they need (forward: one per k
  // slot, 16 for both substeps; dX: one per column block).
  // Per tile and lane: dX -- nib[b][j] = 8 codes (k slots 32 h2 + 8 (2 kh +
  // j) + 0..7) of column block b and sc[b] its scale; forward -- nib[j][w] =
  // codes of columns 16 seg + 8 w .. +7 of k row kr(j) and sc[j] its scale.
  constexpr int kNS = 2;
  auto read_tile = [&](const char *st, uint32_t (&nib)[2][2], float (&sc)[kNS]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const i32x2_t v = *reinterpret_cast<const i32x2_t *>(st + kXBytes + co[b]);
      nib[b][0] = uint32_t(v[0]);
      nib[b][1] = uint32_t(v[1]);
    }
    const char *sp = st + kXBytes + kCBytes + so;
    if constexpr (kFwd) {
      sc[0] = *reinterpret_cast<const float *>(sp);
      sc[1] = *reinterpret_cast<const float *>(sp + 32);     // k row kr(1) = kr(0) + 8
    } else {
      const float s0 = *reinterpret_cast<const float *>(sp);
      const float s1 = *reinterpret_cast<const float *>(sp + 128);
      sc[0] = kh ? s1 : s0;                                  // accumulator b = column block b ^ kh
      sc[1] = kh ? s0 : s1;
    }
  };
  auto read_a = [&](const char *st, int j, u32x4_t (&a)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const u32x4_t *>(st + xo[j] + 4096 * i);
  };
  // dX: one scale per column block and tile, so the expansion goes through a
  // per-scale table built at substep 0 and reused at substep 1.
  ScaledTable tbl[2];
  // dX: the expansion of substep j of a tile, in registers (per-scale
  // tables built at substep 0 and reused at substep 1).
  auto make_b = [&](const uint32_t (&nib)[2][2], const float (&sc)[kNS], int j, u32x4_t (&bb)[2]) {
    if (j == 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b) tbl[b] = scaled_table(sc[b], tb);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) bb[b] = expand8_table(nib[b][j], tbl[b]);
  };
  // Forward: this lane's 16 weights of one k row (one scale) of substep j,
  // expanded into the wavefront's scratch ...
  auto expand_write = [&](const uint32_t (&nib)[2][2], const float (&sc)[kNS], int j) {
    const ScaledTable T = scaled_table(sc[j], tb);
    const u32x4_t w0 = expand8_table(nib[j][0], T), w1 = expand8_table(nib[j][1], T);
    *reinterpret_cast<u32x4_t *>(scr + swo) = w0;
    *reinterpret_cast<u32x4_t *>(scr + swo + 16) = w1;
  };
  // ... and read back transposed as the two B fragments.
  auto read_b = [&](u32x4_t (&bb)[2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) bb[b] = lds_col8_32<kXPitch>(scr, 32 * (b ^ kh));   // see the epilogue
  };
  auto mfmas = [&](const u32x4_t (&a)[8], const u32x4_t (&bb)[2]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[b][i] = mfma32x32x16(a[i], bb[b], acc[b][i]);
  };

  // dB fold.  XA^T of the workgroup's 256 tokens (8 KiB bf16) goes to the
  // LDS area the forward uses as expansion scratch, by direct-to-LDS loads
  // issued before the prologue's (so its first wait covers them): row j =
  // rank j (512 B), 16-B token chunk t stored in slot t ^ j so that the 16
  // ranks of one chunk read from distinct banks.  A operand of the
  // 16 x 16 x 32 products: lane = rank j (lane & 15), tokens 32 s + 8 g ..
  // + 7 (g = lane >> 4), i.e. chunk 4 s + g.  B operand: lane i16 = 4 tq + q
  // of group g points at dY row 32 s + 8 g + tq (+ 4), columns 16 w + 4 q ..
  // + 3 (16-B chunk 2 w + (q >> 1), half q & 1); the row swizzle does not
  // depend on s, so the eight steps are fixed offsets 4096 s from two
  // per-lane offsets.  Lane results: ranks 4 g .. 4 g + 3 of dB column
  // 64 kt + 16 w + i16.
  int db_first = KT;                // first tile whose dB columns this workgroup forms
  uint32_t db_lo = 0, db_hi = 0, db_a = 0;
  uint32_t db_off = kNoStore;       // byte offset of this lane's results for tile 0
  f32x4_t db_res[kMaxDbTiles];
  char *const sxat = smem + kRingBytes;
  if constexpr (!kFwd) {
    if (dbf.part) {
      const rsrc_t rA = make_rsrc(dbf.xat, 16 * dbf.ldm * 2);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int j = 2 * (2 * wave + p) + (lane >> 5), t = (lane & 31) ^ j;
        lds_load16(rA, lds_addr(sxat) + (2 * wave + p) * 1024,
                   uint32_t((j * dbf.ldm + m0 + 8 * t) * 2), 0u);
      }
      const int i16 = lane & 15, g = lane >> 4, q = i16 & 3, tq = i16 >> 2;
      db_first = __builtin_amdgcn_readfirstlane(int(n0 / BN) < KT ? int(n0 / BN) : KT);
      db_a = uint32_t(i16 * 512 + 16 * (g ^ i16));    // + 64 s: chunk (4 s + g) ^ i16
      const int c = 2 * wave + (q >> 1);
      db_lo = xoff(8 * g + tq, c) + 8 * (q & 1);
      db_hi = xoff(8 * g + tq + 4, c) + 8 * (q & 1);
      if (4 * g < dbf.r)                              // ranks past r: nothing to store
        db_off = uint32_t((((m0 / BM) * K + 16 * wave + i16) * dbf.r + 4 * g) * 4);
    }
  }
  auto db_tile = [&](const char *st) {
    u32x4_t xa[8], bt[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      xa[s] = *reinterpret_cast<const u32x4_t *>(sxat + (db_a ^ uint32_t(64 * s)));
      const u32x2_t lo = lds_tr4(st + db_lo + 4096 * s);
      const u32x2_t hi = lds_tr4(st + db_hi + 4096 * s);
      bt[s] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
    return db_chain(xa, bt);
  };

  // ---- prologue: tiles 0..kStages-1 in flight (clamped to the last tile);
  // tiles 0 and 1 landed and visible.
  static_assert(kStages >= 4, "the pipeline keeps two tiles visible ahead of the issue");
#pragma unroll
  for (int p = 0; p < kStages; ++p) issue(p < KT ? p : KT - 1, p);
  wait_vmcnt<(kStages - 2) * kLoadsPerTile>();
  __syncthreads();
  uint32_t nib[2][2], nibn[2][2];
  float sc[kNS], scn[kNS];
  u32x4_t a0[8], a1[8], b0[2], b1[2];

  if constexpr (kFwd) {
    // Forward pipeline.  The scratch holds one substep at a time: in every
    // half-step the B fragments of the next half-step are read from it first,
    // then the substep after that is expanded into it (same wavefront, LDS
    // in order: the reads see the old contents).  Codes of tile kt+2 are read
    // in the second half of iteration kt, one half-step before their first
    // expansion.  Invariant at the top of iteration kt: tiles kt, kt+1
    // visible; a0/b0 = substep 0 of tile kt; scratch = substep 1 of tile kt;
    // nib/sc = codes and scales of tile kt+1.
    read_tile(smem, nib, sc);
    expand_write(nib, sc, 0);
    read_b(b0);
    expand_write(nib, sc, 1);
    read_tile(smem + kStageBytes, nib, sc);
    read_a(smem, 0, a0);
    for (int kt = 0; kt < KT; ++kt) {
      const char *st = smem + (kt % kStages) * kStageBytes;
      const char *sn = smem + ((kt + 1) % kStages) * kStageBytes;
      const char *s2 = smem + ((kt + 2) % kStages) * kStageBytes;
      // substep 0 of tile kt; prepare substep 1 of kt, expand substep 0 of kt+1
      read_a(st, 1, a1);
      read_b(b1);
      expand_write(nib, sc, 0);
      mfmas(a0, b0);
      sched_pattern<12, 6>();        // (10, 4 and 14, 4 below: about 2 % slower)
      // tile kt+2 landed and visible; the stage of tile kt is free
      wait_vmcnt<(kStages - 3) * kLoadsPerTile>();
      __syncthreads();
      issue(kt + kStages < KT ? kt + kStages : KT - 1, kt % kStages);
      // substep 1 of tile kt; prepare substep 0 of kt+1, expand substep 1 of
      // kt+1, fetch the codes of kt+2 (past the end: stages never used)
      read_tile(s2, nibn, scn);
      read_a(sn, 0, a0);
      read_b(b0);
      expand_write(nib, sc, 1);
      mfmas(a1, b1);
      sched_pattern<16, 6>();
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        nib[b][0] = nibn[b][0];
        nib[b][1] = nibn[b][1];
      }
#pragma unroll
      for (int q = 0; q < kNS; ++q) sc[q] = scn[q];
    }
  } else {
    // dX pipeline.  Invariant at the top of iteration kt: tiles kt and kt+1
    // are visible; a0/b0 hold substep 0 of tile kt and nib/sc its codes and
    // scales.  Codes and scales are read one half-step before they are
    // expanded, so no expansion waits on LDS.
    auto body = [&](int kt) {
      const char *st = smem + (kt % kStages) * kStageBytes;
      const char *sn = smem + ((kt + 1) % kStages) * kStageBytes;
      // substep 0 of tile kt; prepare substep 1 and fetch tile kt+1's codes
      read_tile(sn, nibn, scn);
      read_a(st, 1, a1);
      make_b(nib, sc, 1, b1);
      mfmas(a0, b0);
      sched_pattern<12, 6>();
      // tile kt+2 landed and visible; the stage of tile kt is free
      wait_vmcnt<(kStages - 3) * kLoadsPerTile>();
      __syncthreads();
      issue(kt + kStages < KT ? kt + kStages : KT - 1, kt % kStages);
      // substep 1 of tile kt; prepare substep 0 of tile kt+1 (past the end:
      // reads of a stage that is never used)
      read_a(sn, 0, a0);
      make_b(nibn, scn, 0, b0);
      mfmas(a1, b1);
      sched_pattern<8, 6>();
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        nib[b][0] = nibn[b][0];
        nib[b][1] = nibn[b][1];
      }
#pragma unroll
      for (int q = 0; q < kNS; ++q) sc[q] = scn[q];
    };
    read_tile(smem, nib, sc);
    read_a(smem, 0, a0);
    make_b(nib, sc, 0, b0);
    // The K loop runs in segments that end at the workgroup's dB tiles: the
    // dB columns of tile d are formed at the top of iteration d (its stage
    // visible, freed only by that iteration's barrier), between two runs of
    // the unbranched loop body, and held in registers until the loop is over,
    // so that no store enters the loop's vmcnt waits.
    // (kt and the segment ends are uniform; readfirstlane keeps them scalar)
    int kt = 0;
#pragma unroll
    for (int i = 0; i < kMaxDbTiles; ++i) {
      const int d = __builtin_amdgcn_readfirstlane(db_first + i * dbf.ncw);
      const int e = d < KT ? d : KT;
      for (; kt < e; ++kt) body(kt);
      kt = __builtin_amdgcn_readfirstlane(kt);
      db_res[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (d < KT) db_res[i] = db_tile(smem + (d % kStages) * kStageBytes);
    }
    for (; kt < KT; ++kt) body(kt);
  }
  wait_vmcnt<0>();
  if constexpr (!kFwd) {
    if (db_off != kNoStore) {
#pragma unroll
      for (int i = 0; i < kMaxDbTiles; ++i) {
        const int d = db_first + i * dbf.ncw;
        if (d < KT)
          *reinterpret_cast<f32x4_t *>(reinterpret_cast<char *>(dbf.part) + db_off +
                                       int64_t(d) * BK * dbf.r * 4) = db_res[i];
      }
    }
  }
}

// The adapter factor of the rank-r term, read in the caller's layout and
// dtype: element (n, j) = Q[n * sn + j * sj] for j < r, 0 beyond.
struct AdapterRef {
  const void *Q;
  bool bf16;
  int64_t sn, sj;
  int r;
};

// 8 consecutive rank indices j0..j0+7 of row n of the adapter factor, as
// loaded (bf16 or fp32 bits): the loads go out back to back with no
// condition around them (an element past the row or past r loads element 0
// and is zeroed when packed), so no wait comes between them; pack8 turns
// them into the bf16x8 MFMA operand at the point of use.
struct Adapter8 {
  uint16_t h[8];     // bf16 adapters
  uint32_t v[8];     // fp32 adapters
};

__device__ __forceinline__ Adapter8 load_adapter8(const AdapterRef &q, int64_t n, bool row_ok,
                                                  int j0) {
  Adapter8 a;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    a.h[t] = 0;
    a.v[t] = 0;
  }
  if (q.bf16) {
    const uint16_t *p = static_cast<const uint16_t *>(q.Q);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int j = j0 + t;
      a.h[t] = p[(row_ok && j < q.r) ? n * q.sn + int64_t(j) * q.sj : 0];
    }
  } else {
    const uint32_t *p = static_cast<const uint32_t *>(q.Q);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int j = j0 + t;
      a.v[t] = p[(row_ok && j < q.r) ? n * q.sn + int64_t(j) * q.sj : 0];
    }
  }
  return a;
}

__device__ __forceinline__ u32x4_t pack8(const AdapterRef &q, const Adapter8 &a, bool row_ok,
                                         int j0) {
  uint32_t e[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t v = q.bf16 ? uint32_t(a.h[t]) : uint32_t(bf16_bits(__uint_as_float(a.v[t])));
    e[t] = (row_ok && j0 + t < q.r) ? v : 0u;
  }
  return u32x4_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
}

// Operands of 16 rank indices r0 .. r0 + 15 of the rank-r term, as loaded:
// p[i] = P16 rows m0 + 32 i + l32, ranks r0 + 8 h2 .. +7 (rows past M load
// row 0 and are zeroed at use); qa[b] = adapter rows nw + 32 b + l32, the
// same ranks.  The first 16 are loaded when the kernel starts (independent
// of the K loop), with no wait, so that the epilogue does not wait for them.
struct RankOps {
  u32x4_t p[8];
  Adapter8 qa[2];
};

__device__ __forceinline__ void load_rank_ops(RankOps &o, const uint16_t *__restrict__ P16, int ldp,
                                              const AdapterRef &q, int r0, int64_t M, int64_t N,
                                              int64_t m0, int64_t nw) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, h2 = lane >> 5;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t n = nw + 32 * b + l32;
    o.qa[b] = load_adapter8(q, n, n < N, r0 + 8 * h2);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + 32 * i + l32;
    o.p[i] = *reinterpret_cast<const u32x4_t *>(P16 + (m < M ? m : 0) * ldp + r0 + 8 * h2);
  }
}

// The rank-r products of one RankOps into acc.
__device__ __forceinline__ void rank_mfmas(f32x16_t (&acc)[2][8], const RankOps &o,
                                           const AdapterRef &q, int r0, int64_t M, int64_t N,
                                           int64_t m0, int64_t nw) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, h2 = lane >> 5;
  u32x4_t qb[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) qb[b] = pack8(q, o.qa[b], nw + 32 * b + l32 < N, r0 + 8 * h2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const u32x4_t pi = m0 + 32 * i + l32 < M ? o.p[i] : zero;
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[b][i] = mfma32x32x16(pi, qb[b], acc[b][i]);
  }
}

// Epilogue.  The rank-r term P16 . Q^T (P16 bf16 [M x ldp], zero-padded
// columns r..ldp-1; Q the adapter factor, rows indexed by the output column)
// is added by the k-half-0 wavefronts only, so it enters every output once
// (ranks 0..15 from operands loaded at kernel start).  Both K loops keep
// column block b ^ kh in accumulator b, so in every wavefront acc[0] is the
// column block it finishes (kh) and acc[1] the one its partner (the other k
// half) finishes; for kh = 0 that is the plain order, so the rank-r term
// needs no change.  The k halves then meet in two rounds of four row blocks:
// a wavefront writes
// acc[1] of row blocks 4 h .. 4 h + 3 (16 KiB; 64 KiB in all), adds the
// partner's copy of its own block to acc[0] (p0 + p1 either way round: fp32
// addition commutes, so the bits are the four-round epilogue's), stages the
// sums row-major and, after a barrier, stores half of the 128 staged rows
// as whole row segments.  LDS layout per fragment: 4 chunks of 1 KiB, chunk
// c = registers 4c..4c+3 of every lane (16 B per lane, contiguous across
// lanes).  (Exchanging both blocks in four rounds took twice the LDS
// traffic and twelve barriers.)  The row segments leave with non-temporal
// stores (1 us less per launch at 2048 x 4096 x 4096 than cached stores).
template <bool kOutBf16>
__device__ __forceinline__ void epilogue(f32x16_t (&acc)[2][8], char *smem, const RankOps &ro,
                                          const uint16_t *__restrict__ P16, int ldp,
                                          const AdapterRef q, int64_t M,
                                          int64_t N, int64_t m0, int64_t n0, void *__restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ch = wave & 1, kh = wave >> 1;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int64_t nw = n0 + 64 * ch;

  if (kh == 0 && q.r > 0) {
    rank_mfmas(acc, ro, q, 0, M, N, m0, nw);
    for (int r0 = 16; r0 < q.r; r0 += 16) {
      RankOps o;
      load_rank_ops(o, P16, ldp, q, r0, M, N, m0, nw);
      rank_mfmas(acc, o, q, r0, M, N, m0, nw);
    }
  }

  constexpr int kOE = kOutBf16 ? 2 : 4;                       // output element bytes
  constexpr int kOPitch = kOutBf16 ? 144 : 272;               // staging row pitch (bytes)
  static_assert(65536 + 2 * 128 * kOPitch <= Geo<false>::kLdsBytes, "epilogue LDS");
  char *stg = smem + 65536 + ch * 128 * kOPitch;              // 128 rows x 64 columns per ch
  char *wr = smem + (ch * 2 + kh) * 16384 + lane * 16;        // this wavefront's region
  const char *rd = smem + (ch * 2 + (1 - kh)) * 16384 + lane * 16;   // the partner's
  const bool ncol = nw < N;                                   // N % 64 == 0
  auto round = [&](auto H) {
    constexpr int h = decltype(H)::value;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const f32x16_t v = acc[1][4 * h + f];
      char *w = wr + f * 4096;
      *reinterpret_cast<f32x4_t *>(w) = __builtin_shufflevector(v, v, 0, 1, 2, 3);
      *reinterpret_cast<f32x4_t *>(w + 1024) = __builtin_shufflevector(v, v, 4, 5, 6, 7);
      *reinterpret_cast<f32x4_t *>(w + 2048) = __builtin_shufflevector(v, v, 8, 9, 10, 11);
      *reinterpret_cast<f32x4_t *>(w + 3072) = __builtin_shufflevector(v, v, 12, 13, 14, 15);
    }
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t *>(rd + f * 4096 + c * 1024);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[0][4 * h + f][4 * c + e] + x[e];
          const int row = 32 * f + 8 * c + 4 * h2 + e;        // register 4c + e
          char *d = stg + row * kOPitch + (32 * kh + l32) * kOE;
          if constexpr (kOutBf16)
            *reinterpret_cast<uint16_t *>(d) = bf16_bits(v);
          else
            *reinterpret_cast<float *>(d) = v;
        }
      }
    }
    __syncthreads();
    // wavefront kh stores staged rows 64 kh .. 64 kh + 63 of these 128
    constexpr int kChunks = 64 * kOE / 16;                    // 16-B chunks per row
#pragma unroll
    for (int qq = 0; qq < kChunks; ++qq) {
      const int cid = lane + 64 * qq;
      const int row = 64 * kh + cid / kChunks, c = cid % kChunks;
      const int64_t m = m0 + 128 * h + row;
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stg + row * kOPitch + 16 * c);
      if (ncol && m < M)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(static_cast<char *>(Y) + (m * N + nw) * kOE + 16 * c));
    }
  };
  // Round 0 follows the K loop's last LDS reads; round 1's exchange writes
  // follow round 0's exchange reads (two barriers back) and its staging
  // writes follow round 0's stores (one barrier back).
  __syncthreads();
  round(std::integral_constant<int, 0>{});
  round(std::integral_constant<int, 1>{});
}

// ================================================================ forward
template <bool kOutBf16, bool kG16>
__global__ __launch_bounds__(kThreads, 1) void fwd_gemm_kernel(
    const uint8_t *__restrict__ codes, const float *__restrict__ cs, int64_t K, int64_t N,
    const uint16_t *__restrict__ X16, int64_t M, const uint16_t *__restrict__ XA16,
    int ldp, AdapterRef bq, void *__restrict__ Y, ExpandConsts tb,
    int nt_count) {
  extern __shared__ __align__(16) char smem[];
  int mt, nt;
  tile_of(nt_count, mt, nt);
  const int64_t m0 = int64_t(mt) * BM, n0 = int64_t(nt) * BN;
  RankOps ro;
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 2 && bq.r > 0)  // k-half-0 wavefronts
    load_rank_ops(ro, XA16, ldp, bq, 0, M, N, m0, n0 + 64 * ((threadIdx.x >> 6) & 1));
  f32x16_t acc[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[b][i][r] = 0.f;
  gemm_mainloop<true, kG16>(X16, M, K, N, codes, cs, m0, n0, tb, smem, acc, DbFold{});
  // rank-r term: y += XA16 . B (B read as rows n of B^T)
  epilogue<kOutBf16>(acc, smem, ro, XA16, ldp, bq, M, N, m0, n0, Y);
}

// ================================================================ dX
template <bool kOutBf16, bool kG16>
__global__ __launch_bounds__(kThreads, 1) void dx_gemm_kernel(
    const uint8_t *__restrict__ codes, const float *__restrict__ cs, int64_t IN, int64_t OUT,
    const uint16_t *__restrict__ dY16, int64_t M, const uint16_t *__restrict__ G16,
    int ldp, AdapterRef aq, void *__restrict__ dX, ExpandConsts tb,
    int nt_count, DbFold dbf) {
  extern __shared__ __align__(16) char smem[];
  int mt, nt;
  tile_of(nt_count, mt, nt);
  const int64_t m0 = int64_t(mt) * BM, i0 = int64_t(nt) * BN;
  RankOps ro;
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 2 && aq.r > 0)
    load_rank_ops(ro, G16, ldp, aq, 0, M, IN, m0, i0 + 64 * ((threadIdx.x >> 6) & 1));
  f32x16_t acc[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[b][i][r] = 0.f;
  gemm_mainloop<false, kG16>(dY16, M, OUT, IN, codes, cs, m0, i0, tb, smem, acc, dbf);
  // rank-r term: dX += G16 . A^T (A read as rows i of A)
  epilogue<kOutBf16>(acc, smem, ro, G16, ldp, aq, M, IN, m0, i0, dX);
}

bool set_lds(const void *fn, int bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) ==
         hipSuccess;
}

}  // namespace

hipError_t launch_fwd_gemm(const uint8_t *codes, const float *cs, int64_t K, int64_t N,
                           const uint16_t *X16, int64_t M, const uint16_t *XA16, int32_t ldp,
                           const void *B, bool b_bf16, int32_t r, void *Y, bool y_bf16,
                           int codebook, bool g16, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const AdapterRef bq{B, b_bf16, 1, N, int(r)};
  const int mtc = int((M + BM - 1) / BM), ntc = int((N + BN - 1) / BN);
  dim3 grid(unsigned(mtc * ntc));
  if (!tables(codebook).symmetric) return hipErrorInvalidValue;
  const ExpandConsts tb = tables(codebook).expand;
#define QLORA_FWD(OB, G)                                                                        \
  do {                                                                                          \
    constexpr int lds = Geo<G>::kLdsBytes;                                                      \
    static bool ok = set_lds(reinterpret_cast<const void *>(&fwd_gemm_kernel<OB, G>), lds);     \
    if (!ok) return hipErrorInvalidValue;                                                       \
    hipLaunchKernelGGL((fwd_gemm_kernel<OB, G>), grid, dim3(kThreads), lds, s, codes, cs, K, N, \
                       X16, M, XA16, int(ldp), bq, Y, tb, ntc);                                 \
  } while (0)
  if (g16) {
    if (y_bf16) QLORA_FWD(true, true);
    else QLORA_FWD(false, true);
  } else {
    if (y_bf16) QLORA_FWD(true, false);
    else QLORA_FWD(false, false);
  }
#undef QLORA_FWD
  return hipGetLastError();
}

bool dx_fold_fits(int64_t M, int64_t in, int64_t out) {
  const int64_t ncw = (in + BN - 1) / BN, kt = out / BK;
  return M > 0 && (kt + ncw - 1) / ncw <= kMaxDbTiles;
}

hipError_t launch_dx_gemm(const uint8_t *codes, const float *cs, int64_t in, int64_t out,
                          const uint16_t *dY16, int64_t M, const uint16_t *G16, int32_t ldp,
                          const void *A, bool a_bf16, int32_t r, void *dX, bool dx_bf16,
                          int codebook, bool g16, const uint16_t *xat, int64_t ldm,
                          float *db_part, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const AdapterRef aq{A, a_bf16, int64_t(r), 1, int(r)};
  const int mtc = int((M + BM - 1) / BM), ntc = int((in + BN - 1) / BN);
  // the XA^T fragments of the last token block reach token mtc * 256 - 1
  if (db_part && (!xat || r < 1 || r > 16 || r % 4 != 0 || ldm < int64_t(mtc) * BM))
    return hipErrorInvalidValue;
  const DbFold dbf{xat, ldm, db_part, int(r), ntc};
  if (db_part && (!dx_fold_fits(M, in, out) || int64_t(mtc) * out * r * 4 > 0x7fffffff))
    return hipErrorInvalidValue;
  dim3 grid(unsigned(mtc * ntc));
  if (!tables(codebook).symmetric) return hipErrorInvalidValue;
  const ExpandConsts tb = tables(codebook).expand;
#define QLORA_DX(OB, G)                                                                         \
  do {                                                                                          \
    constexpr int lds = Geo<G>::kLdsBytes;                                                      \
    static bool ok = set_lds(reinterpret_cast<const void *>(&dx_gemm_kernel<OB, G>), lds);      \
    if (!ok) return hipErrorInvalidValue;                                                       \
    hipLaunchKernelGGL((dx_gemm_kernel<OB, G>), grid, dim3(kThreads), lds, s, codes, cs, in,    \
                       out, dY16, M, G16, int(ldp), aq, dX, tb, ntc, dbf);                      \
  } while (0)
  if (g16) {
    if (dx_bf16) QLORA_DX(true, true);
    else QLORA_DX(false, true);
  } else {
    if (dx_bf16) QLORA_DX(true, false);
    else QLORA_DX(false, false);
  }
#undef QLORA_DX
  return hipGetLastError();
}

}  // namespace qlora
