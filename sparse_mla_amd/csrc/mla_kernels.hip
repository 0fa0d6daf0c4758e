// HIP kernels of the absorbed sparse MLA decode step, written for CDNA4
// (gfx950): 64-wide wavefronts, bf16 MFMA 32x32x16, LDS transpose reads and
// buffer loads that write straight into LDS.
//
// Operation (DeepSeek-V3.2-Exp pages, decode mode):
//   absorb   q~ = q_nope W_UK,h          "Query-key similarity" page, code excerpt
//   decode   s = scale (q~ c^T + q_pe k_pe^T) on the selected rows, softmax over
//            keys, O~ = A c                "Query-key similarity" page, formula
//            S_i and index mask; "Softmax" page, formula for A
//   combine  log-sum-exp merge of key-split partials
//   value-up O = O~ W_UV,h^T               "Apply value weights" page, formula O_i
//
// MFMA operand layout used throughout (v_mfma_f32_32x32x16_bf16, lane l,
// v = 0..7 for A/B, 0..15 for C):
//   A[m][k]: m = l % 32, k = 8 (l / 32) + v
//   B[k][n]: n = l % 32, k = 8 (l / 32) + v
//   C[m][n]: m = 8 (v / 4) + 4 (l / 32) + v % 4, n = l % 32
// Any permutation of k applied to both A and B leaves the product unchanged,
// which the decode kernel uses to feed P straight from the score registers.
//
// ds_read_b64_tr_b16: within each 16-lane group, output lane j element e is
// element (j % 4) of the 8 bytes addressed by source lane 4 e + j / 4.  With
// source lane i addressing row r0 + i / 4, columns c0 + 4 (i % 4) .. + 3 of a
// row-major tile, lane j receives column c0 + j of rows r0 .. r0 + 3: a
// K-strided operand fragment.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>
#include <math.h>
#include <stdint.h>

#include "mla_kernels.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLn2 = 0.69314718055994530942f;
// Lazy rescaling of the running softmax state: the reference maximum moves
// only when a block's maximum exceeds it by more than this (log2 units), so
// probabilities stay <= 2^8 and the accumulators are rescaled rarely.
constexpr float kRescaleLog2 = 8.0f;
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw buffer, 32-bit data format
constexpr uint32_t kMaskedOffset = 0x80000000u; // beyond every record range: loads 0

// 16-byte position swizzle inside a 128-byte LDS segment, from key bits b0..b3:
// (b2, b1, b0 ^ b1 ^ b3).
__device__ __forceinline__ uint32_t seg_swz(uint32_t key) {
  return ((key >> 2) & 1u) | (key & 2u) | (((key ^ (key >> 1) ^ (key >> 3)) & 1u) << 2);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource: 48-bit base, stride 0, num_records bytes, 32-bit data
// format.  Loads at offsets >= num_records return zeros.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t num_records) {
  const uint64_t addr = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
  r[3] = (int)kBufferFlags;
  return r;
}

// 16 bytes per lane from buffer offset `voff` straight into LDS at
// lds_base + 16 * lane (buffer_load_dwordx4 ... lds, LDS base in M0).
// Written as asm so that the compiler does not treat every later LDS read as
// a possible alias of the in-flight load and wait for all of them; the
// kernel orders these loads itself with s_waitcnt vmcnt and a barrier.  The
// instruction has no destination register.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// The same with 4 bytes per lane (lane l lands at lds_base + 4 l).
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Score-chain MFMAs with the accumulator in VGPRs.  The kernels that use
// them keep their big accumulators in AGPRs (AGPR-form compiler MFMAs), and a
// compiler MFMA would put this chain there too.
// Back-to-back accumulation into the same registers needs no wait states;
// a vector read of the result does, so the last MFMA of a chain is
// mfma32_v_last.  Inline asm hides the MFMA's latency from the compiler,
// which takes the result as written when the statement ends: code around a
// chain must give the compiler no reason to copy the accumulator between two
// of its MFMAs (such a copy would read a sum still in flight).  Wait states
// after every MFMA would rule that out, but they stall the wave's issue
// behind the matrix pipe and roughly double the chain's time.
// mfma32_v also takes the previous chain MFMA's A operand (`keep`, unused):
// that register then stays allocated until this dependent MFMA issues, so
// the compiler puts no vector result in it while the matrix core may still
// be reading it (the write would wait for the read to finish).
__device__ __forceinline__ f32x16 mfma32_v_first(bf16x8 a, bf16x8 b) {
  f32x16 c;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  return c;
}
__device__ __forceinline__ void mfma32_v(f32x16& c, bf16x8 a, bf16x8 b, bf16x8 keep) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b), "v"(keep));
}
__device__ __forceinline__ void mfma32_v_last(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7"
               : "+v"(c)
               : "v"(a), "v"(b));
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero8() {
  i16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
  return __builtin_bit_cast(bf16x8, z);
}

// Two transpose reads (k-rows r and r + 4 of a fragment) joined into one
// 8-element MFMA operand.
__device__ __forceinline__ bf16x8 tr_pair(const char LDS_AS* p0, const char LDS_AS* p1) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)p0);
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)p1);
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Four floats -> four bf16 (round to nearest even), packed for an 8-byte
// store; each pair is one two-input conversion.
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return uint2{pack2(a, b), pack2(c, d)};
}

// ---------------------------------------------------------------------------
// fp8 dequantisation: E4M3FN from its definition (sign, 4 exponent bits with
// bias 7, 3 mantissa bits; exponent 0 is subnormal, m/8 * 2^-6; 0x7F / 0xFF
// are NaN).  The product with the fp32 block scale is rounded to bf16 from
// its exact value: p = fl(v * s) plus the exact residual fma(v, s, -p)
// decide the ties that fl() can create.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t e = (code >> 3) & 15u, m = code & 7u;
  float v;
  if (e == 0u) v = (float)m * 0x1p-9f;
  else if (e == 15u && m == 7u) v = __builtin_nanf("");
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (code & 0x80u) ? -v : v;
}

__device__ __forceinline__ uint32_t bf16_rne_exact(float p, float err) {
  const uint32_t u = __float_as_uint(p);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  const uint32_t lower = u & 0xffffu, hi = u >> 16;
  bool up;
  if (lower > 0x8000u) up = true;
  else if (lower < 0x8000u) up = false;
  else if (err == 0.f) up = (hi & 1u) != 0u;
  else up = (err > 0.f) == (p > 0.f);   // the exact value lies beyond the tie
  return hi + (up ? 1u : 0u);
}

// Two fp8 codes (bytes 0-1 of `word`, or 2-3 with HI) times the block
// scale, rounded to bf16, packed.  The hardware conversion decodes the codes
// exactly.  Rounding the fp32 product fl(v * s) to bf16 equals rounding the
// exact product except where fl(v * s) sits exactly on a bf16 tie (low 16
// bits 0x8000) with a nonzero residual: EXACT settles every pair by the exact
// rule above; otherwise the packed round-to-nearest-even conversion is used,
// for blocks that block_has_ties() clears.  A NaN code gives a bf16 NaN.
template <bool HI, bool EXACT>
__device__ __forceinline__ uint32_t dq_pair(uint32_t word, float s) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
  const float p0 = v[0] * s, p1 = v[1] * s;
  if constexpr (EXACT)
    return bf16_rne_exact(p0, __builtin_fmaf(v[0], s, -p0)) | (bf16_rne_exact(p1, __builtin_fmaf(v[1], s, -p1)) << 16);
  return pack2(p0, p1);
}
// Eight codes (two words) -> eight bf16 values as an MFMA operand.
template <bool EXACT>
__device__ __forceinline__ bf16x8 dq8(uint2 codes, float s) {
  const uint4 w = uint4{dq_pair<false, EXACT>(codes.x, s), dq_pair<true, EXACT>(codes.x, s),
                        dq_pair<false, EXACT>(codes.y, s), dq_pair<true, EXACT>(codes.y, s)};
  return __builtin_bit_cast(bf16x8, w);
}
// Whether some code, times the block scale s, has its fp32 product on a bf16
// tie with a nonzero residual -- the only products whose bf16 rounding needs
// the exact rule.  Wave-uniform: each lane tests four of the 256 codes.
__device__ __forceinline__ bool block_has_ties(float s, int lane) {
  bool t = false;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float v = __builtin_amdgcn_cvt_f32_fp8(lane + 64 * k, 0);
    const float p = v * s;
    t |= ((__float_as_uint(p) & 0xffffu) == 0x8000u) && (__builtin_fmaf(v, s, -p) != 0.f);
  }
  return __builtin_amdgcn_ballot_w64(t) != 0;
}

// ---------------------------------------------------------------------------
// absorb: q_abs[b][h][c] = sum_d q_nope[b][h][d] W_UK,h[d][c]
// Workgroup = (head, 256-column half): 256 workgroups, each streaming its
// 64 KB slab of W_UK once.  W_UK is stored [d][c] (c contiguous) while d is
// the reduction index, so the 128 x 256 slab is moved into LDS by LDS-DMA --
// 8 lanes per 128-byte line, line m (64 columns) of row d at segment
// (m * 128 + d), chunk q at 16-byte position q ^ 2 (d % 4), which keeps the
// transpose reads conflict-free -- and read back as K-strided MFMA
// fragments.  The half is done as two 128-column quarters (lines 0-1, then
// 2-3), each a 32 KB region: the first quarter's products and stores run
// while the second quarter's slab is still arriving.  In quarter Q wave w
// owns columns 128 Q + 32 w .. + 31: M = c, N = b, K = d.
// The query rows (B operand) also come by LDS-DMA, four 32-row batch tiles
// at a time, laid out like a gathered block of the decode (row r of a tile,
// line m = d / 64 at m * 4 KB + r * 128, chunk swizzled by seg_swz(r)), so
// each load moves whole lines; read directly, each would touch 32 rows for
// 32 bytes apiece.  Two sets of four tiles alternate: with more than 128
// batch rows the next group's tiles arrive while the current group's
// products and stores run.  With no compiler-visible load, every wait is
// explicit.
// ---------------------------------------------------------------------------
constexpr int kAbsQ = 32 * 1024;             // one quarter of the slab
constexpr int kAbsQTile = 2 * 32 * 128;      // one 32-row query tile (8 KB)
constexpr int kAbsLds = 2 * kAbsQ + 8 * kAbsQTile;

// With FP8 the slab is read as block-scaled fp8 codes (32 KB per half, one
// scale per quarter: its 128 rows and 128 columns are one scale block) by
// ordinary 16-byte loads into registers and dequantised to bf16 straight into
// the same swizzled LDS layout; the loads of both quarters go out first and
// each quarter is converted when its products need it.
template <bool FP8>
__global__ __launch_bounds__(256) void absorb_kernel(const AbsorbArgs a) {
  __shared__ __attribute__((aligned(1024))) char wt[kAbsLds];
  const int h = (int)blockIdx.x % a.H;
  const int ch = (int)blockIdx.x / a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, i16 = lane & 15, gm = (lane >> 4) & 1;
  const char LDS_AS* wl = (const char LDS_AS*)wt;
  const uint32_t lds0 = (uint32_t)(uintptr_t)wl;
  const uint32_t qt0 = lds0 + (uint32_t)(2 * kAbsQ);  // query tiles

  // Quarter Q of the slab: lines 2Q and 2Q + 1, 32 instructions, 8 per wave.
  const i32x4 rw = buffer_rsrc(a.wkv_b + (size_t)h * kRowsPerHead * kLatent + ch * 256,
                               (uint32_t)((kNope - 1) * kLatent * 2 + 512));
  auto stage_slab = [&](int Q) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int qi = 8 * wave + k;                      // 0 .. 31
      const int m = 2 * Q + (qi >> 4), rg = qi & 15;     // line, row group
      const uint32_t d = (uint32_t)((rg << 3) + (lane >> 3));
      const uint32_t q = (uint32_t)(lane & 7) ^ (2u * (d & 3u));
      dma16(rw, lds0 + (uint32_t)(m * 128 + 8 * rg) * 128u, d * (uint32_t)(kLatent * 2) + (uint32_t)m * 128u + q * 16u);
    }
  };
  // fp8 slab, quarter Q: thread t takes rows d = (t + 256 k) / 8 and 16
  // columns 16 g, g = t % 8, of the quarter (4 loads of 16 codes).
  auto load_slab8 = [&](int Q, uint4 (&raw)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + 256 * k, d = i >> 3, g = i & 7;
      raw[k] = *reinterpret_cast<const uint4*>(a.fp8.w_fp8 + ((size_t)h * kRowsPerHead + d) * kLatent + ch * 256 +
                                               128 * Q + 16 * g);
    }
  };
  // The two quarters' scales and whether either needs the exact rounding
  // rule (read first: nothing else is in flight yet).
  float qsc[2] = {0.f, 0.f};
  bool qtie[2] = {false, false};
  if constexpr (FP8) {
#pragma unroll
    for (int Q = 0; Q < 2; ++Q) {
      qsc[Q] = a.fp8.w_scale[(2 * h) * (kLatent / 128) + 2 * ch + Q];
      qtie[Q] = block_has_ties(qsc[Q], lane);
    }
  }
  auto store_slab8 = [&](int Q, const uint4 (&raw)[4]) __attribute__((always_inline)) {
    const float sc = qsc[Q];
    const bool exact = qtie[Q];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + 256 * k, d = i >> 3, g = i & 7;
      bf16x8 lo, hi;
      if (__builtin_expect(exact, 0)) {
        lo = dq8<true>(uint2{raw[k].x, raw[k].y}, sc);
        hi = dq8<true>(uint2{raw[k].z, raw[k].w}, sc);
      } else {
        lo = dq8<false>(uint2{raw[k].x, raw[k].y}, sc);
        hi = dq8<false>(uint2{raw[k].z, raw[k].w}, sc);
      }
      const uint32_t m = (uint32_t)(2 * Q + (g >> 2));
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t q = (uint32_t)(2 * (g & 3) + c);
        *(bf16x8 LDS_AS*)((char LDS_AS*)wt + (m * 128u + (uint32_t)d) * 128u + ((q ^ (2u * ((uint32_t)d & 3u))) * 16u)) =
            c ? hi : lo;
      }
      if (a.fp8.w_formed != nullptr) {
        uint16_t* f = a.fp8.w_formed + ((size_t)h * kRowsPerHead + d) * kLatent + ch * 256 + 128 * Q + 16 * g;
        *reinterpret_cast<bf16x8*>(f) = lo;
        *reinterpret_cast<bf16x8*>(f + 8) = hi;
      }
    }
  };
  uint4 raw0[4], raw1[4];
  // Query tiles bt0 .. bt0 + 3 (those that exist) into tile set `set`: 8
  // instructions per tile, 2 per wave; rows past B load row B - 1 (their
  // columns are never stored).
  const int nbt = (a.B + 31) / 32;
  auto stage_q = [&](int bt0, int set) __attribute__((always_inline)) {
    const i32x4 rq = buffer_rsrc(a.q_nope + (int64_t)h * a.q_sh, (uint32_t)(((int64_t)(a.B - 1) * a.q_sb + kNope) * 2));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (bt0 + u >= nbt) break;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int qi = 2 * wave + k;                     // 0 .. 7
        const int m = qi >> 2, g = qi & 3;               // line, row group
        const uint32_t r = (uint32_t)(8 * g + (lane >> 3));
        const int bb = min((bt0 + u) * 32 + (int)r, a.B - 1);
        const uint32_t c16 = (((uint32_t)(lane & 7)) ^ seg_swz(r)) * 16u;
        dma16(rq, qt0 + (uint32_t)((4 * set + u) * kAbsQTile + m * 32 * 128 + 8 * g * 128),
              (uint32_t)((int64_t)bb * a.q_sb * 2) + (uint32_t)(m * 128) + c16);
      }
    }
  };
  auto qk_off = [&](int st) __attribute__((always_inline)) -> uint32_t {
    const uint32_t r = (uint32_t)(lane & 31);
    return (uint32_t)((st >> 2) * 32 * 128) + r * 128u + (((uint32_t)(2 * (st & 3) + hh)) ^ seg_swz(r)) * 16u;
  };
  // Slab fragments of quarter Q for this wave (A operand, K-strided).
  auto read_slab = [&](int Q, bf16x8 (&af)[8]) __attribute__((always_inline)) {
    const uint32_t m = (uint32_t)(2 * Q + (wave >> 1));
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      uint32_t off[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint32_t d = (uint32_t)(16 * st + 8 * hh + 4 * r + (i16 >> 2));
        const uint32_t q = (uint32_t)(4 * (wave & 1) + 2 * gm + ((i16 & 3) >> 1));
        off[r] = (m * kNope + d) * 128u + ((q ^ (2u * (d & 3u))) * 16u) + 8u * (uint32_t)(i16 & 1);
      }
      af[st] = tr_pair(wl + off[0], wl + off[1]);
    }
  };
  // Output tile of quarter Q, batch tile bt (staged in the quarter-0 region
  // once its fragments are in registers, two alternating 8 KB buffers): row r
  // (batch row) = 256 bytes, 16-byte chunk c at position c ^ (r % 16).  One
  // barrier per tile: a wave stages tile t + 1 into the buffer of tile t - 1
  // only after the barrier of tile t, which every wave reaches after its
  // copy-out of tile t - 1.
  int ntile = 0;
  auto out_tile = [&](int Q, int bt, const bf16x8 (&af)[8], const bf16x8 (&qb)[8]) __attribute__((always_inline)) {
    f32x16 acc = {};
#pragma unroll
    for (int st = 0; st < 8; ++st) acc = mfma32(af[st], qb[st], acc);
    // acc[v]: batch row lane % 32, column 128 Q + 32 w + 8 (v / 4) + 4 hh + v % 4.
    char* ot = wt + (ntile & 1) * 8192;
    ++ntile;
    char* orow = ot + (lane & 31) * 256 + 8 * hh;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c = 4 * wave + q4;
      *reinterpret_cast<uint2*>(orow + ((c ^ (lane & 15)) << 4)) =
          pack4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
    }
    __syncthreads();
    // Thread t copies chunk t % 16 of rows t / 16 and t / 16 + 16.
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = (tid >> 4) + 16 * k, c = tid & 15;
      const int bb = bt * 32 + r;
      const uint4 val = *reinterpret_cast<const uint4*>(ot + r * 256 + ((c ^ (r & 15)) << 4));
      if (bb < a.B)
        *reinterpret_cast<uint4*>(a.q_abs + ((int64_t)bb * a.H + h) * kLatent + ch * 256 + 128 * Q + 8 * c) = val;
    }
  };

  bf16x8 af0[8], af1[8];
  bf16x8 qb[4][8];
  for (int bt0 = 0; bt0 < nbt; bt0 += 4) {
    const int nq = min(4, nbt - bt0);
    const int set = (bt0 >> 2) & 1;
    if (bt0 == 0) {
      // Quarter 0 of the slab, the first query tiles, quarter 1 of the slab.
      if constexpr (FP8) {
        load_slab8(0, raw0);
        stage_q(0, 0);
        load_slab8(1, raw1);
        store_slab8(0, raw0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        stage_slab(0);
        stage_q(0, 0);
        stage_slab(1);
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      }
    } else {
      // This group's tiles were requested during the previous group: after
      // this wait this wave's have landed, after the barrier every wave's.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (bt0 == 0) read_slab(0, af0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u >= nq) break;
#pragma unroll
      for (int st = 0; st < 8; ++st)
        qb[u][st] = *(const bf16x8 LDS_AS*)(wl + (qt0 - lds0) + (4 * set + u) * kAbsQTile + qk_off(st));
    }
    // The next group's tiles go into the other set, which held the group
    // before this one: every wave read those into registers before the
    // barriers of that group's output tiles, which precede the barrier
    // above.  (The first group requests them only after quarter 1 of the
    // slab has landed, whose wait would otherwise also wait for them.)
    if (bt0 > 0 && bt0 + 4 < nbt) stage_q(bt0 + 4, set ^ 1);
    if (bt0 == 0) {
      // The quarter-0 region holds output tiles from here on.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u >= nq) break;
      out_tile(0, bt0 + u, af0, qb[u]);
    }
    if (bt0 == 0) {
      if constexpr (FP8) store_slab8(1, raw1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      read_slab(1, af1);
      if (4 < nbt) stage_q(4, 1);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u >= nq) break;
      out_tile(1, bt0 + u, af1, qb[u]);
    }
  }
}

// ---------------------------------------------------------------------------
// value-up: out[b][h][d] = sum_c O~[b][h][c] W_UV,h[d][c]
// Workgroup = (head, tile of ROWS batch rows); the tiles of a head run on one
// XCD, so W_UV,h (128 KB, held in registers: wave w keeps value rows
// 32 w .. 32 w + 31) comes from HBM once and from L2 for the other tiles.
// Wave w owns batch rows ROWS/4 * w .. of the tile: it gathers their latent
// rows (one 1 KB row per LDS-DMA instruction, rows past B read as zeros) into
// LDS slots of 1040 bytes, up to 4 splits per pass, and merges them in fp32
// registers; no other wave touches those slots until the merged bf16 tile is
// complete.  Then M = d (W_UV rows), N = b (tile rows from LDS), K = c.
// FUSED: the rows are merged from the split partials of the decode
// ("Softmax" page, normalisation over all selected keys), each the
// unnormalised sum U_s of its split relative to its max m_s:
//   O~ = sum_s g_s U_s, g_s = 2^(m_s - M) / L, L = sum_s 2^(m_s - M) l_s,
//   lse = ln 2 (M + log2 L)
// ---------------------------------------------------------------------------
constexpr int kOtRow = 1040;  // bytes per latent row in LDS (512 bf16 + 16 pad)

// With FP8, W_UV,h is read as block-scaled fp8 codes (8 per lane per K-step,
// in the same issue slots as the bf16 loads) and dequantised to bf16 in
// registers before the products; K-step st lies in scale block column st / 8.
template <bool FUSED, int ROWS, int SPP, bool FP8>
__global__ __launch_bounds__(256, 1) void value_up_kernel(const ValueUpArgs a) {
  __shared__ __attribute__((aligned(1024))) char slots[SPP * ROWS * kOtRow];
  __shared__ float wtab[ROWS * 64];  // merge weights: per wave, row, split
  constexpr int RPW = ROWS / 4;  // batch rows per wave
  // (max, sum) per wave, row and split: the table DMAs write 32 entries
  // each, one DMA when SPP == 2 (at most two splits), up to 2 RPW otherwise.
  constexpr int kMlWave = SPP == 2 ? 32 : RPW * 64;
  __shared__ float2 mltab[FUSED ? 4 * kMlWave : 1];
  static_assert(32 % (SPP * RPW) == 0, "W_UV loads spread evenly over the first merge pass");
  const int ntiles = (a.B + ROWS - 1) / ROWS;
  const int units = a.H * ntiles;
  const int per_xcd = (units + 7) >> 3;
  const int unit = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (unit >= units) return;
  const int h = unit / ntiles, b0 = (unit % ntiles) * ROWS;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrows = min(ROWS, a.B - b0);  // valid rows of the tile
  const int r0 = RPW * wave;              // first tile row of this wave

  const int S = FUSED ? a.S : 1;
  const int64_t sstride = (int64_t)a.B * a.H;  // rows per split
  // fp8: the four scale blocks of W_UV,h (row block 2h + 1) and whether each
  // needs the exact rounding rule, settled before anything else is in flight.
  float wsc[4] = {0.f, 0.f, 0.f, 0.f};
  bool wtie[4] = {false, false, false, false};
  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wsc[j] = a.fp8.w_scale[(2 * h + 1) * (kLatent / 128) + j];
      wtie[j] = block_has_ties(wsc[j], lane);
    }
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(char LDS_AS*)slots;
  const int n = min(RPW, max(0, nrows - r0));  // rows of this wave that exist
  // The wave's own LDS slots hold kCap rows; a pass stages splits
  // c0 .. c0 + ps - 1 of its n rows, split c0 + c row j in slot q = c n + j
  // (slot (q / RPW) ROWS + r0 + q % RPW of the array), so a wave with few
  // rows takes more splits per pass.
  constexpr int kCap = SPP * RPW;
  auto pass_splits = [&](int c0) { return min(S - c0, kCap / max(n, 1)); };
  auto slot_of = [&](int q) { return (q / RPW) * ROWS + r0 + (q % RPW); };
  // Gather one pass: one instruction per (split, row); lane l brings bytes
  // 16 l .. of the row.
  auto gather = [&](int c0) {
    if (n == 0) return;
    const int ps = pass_splits(c0);
    const int64_t row0 = (int64_t)(b0 + r0) * a.H + h;
    for (int c = 0; c < ps; ++c) {
      const uint16_t* base = FUSED ? a.part_o + ((int64_t)(c0 + c) * sstride + row0) * kLatent
                                   : a.o_latent + row0 * kLatent;
      const i32x4 rs = buffer_rsrc(base, (uint32_t)(n - 1) * (uint32_t)a.H * kLatent * 2u + 1024u);
      for (int j = 0; j < n; ++j)
        dma16(rs, lds0 + (uint32_t)(slot_of(c * n + j) * kOtRow),
              (uint32_t)j * (uint32_t)a.H * kLatent * 2u + 16u * (uint32_t)lane);
    }
  };
  // Wait until at most k vector-memory operations are outstanding, k rounded
  // down to a multiple of 8 (waiting longer is always correct).
  auto wait_vm_le = [&](int k) __attribute__((always_inline)) {
    if (k >= 56) asm volatile("s_waitcnt vmcnt(56)" ::: "memory");
    else if (k >= 48) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
    else if (k >= 40) asm volatile("s_waitcnt vmcnt(40)" ::: "memory");
    else if (k >= 32) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
    else if (k >= 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (k >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (k >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // Order of the loads: the (max, sum) of this wave's rows and splits, the
  // first pass of partial rows (split-major), then W_UV,h once the merge
  // weights are computed, spread over the steps of the first merge pass
  // (issued at once, the 32 loads per lane stall the wave's issue until
  // most of them have returned).  vmcnt retires in order, so each split is
  // merged as soon as its rows are in while the later ones still arrive.
  // The (max, sum) come by LDS-DMA too (4 bytes per lane; entry (j G + sp)
  // of the wave's table holds row j, split sp; lanes of splits past S or of
  // rows past the batch land zeros or unused values): a compiler-visible load
  // would get a compiler-placed wait that also drains the partial rows.
  const int G = S <= 1 ? 1 : 1 << (32 - __builtin_clz((unsigned)(S - 1)));
  const int gsh = __builtin_ctz((unsigned)G);
  const int R = 64 >> gsh;
  const int nml = (RPW * 2 * G + 63) >> 6;  // table DMAs: 64 entries each
  float2* mlt = mltab + (FUSED ? wave * kMlWave : 0);
  if constexpr (FUSED) {
    const int64_t bh0 = (int64_t)min(b0 + r0, a.B - 1) * a.H + h;
    const float* mlb = a.part_ml + bh0 * 2;
    const uint32_t rng = (uint32_t)(((int64_t)S * sstride - bh0) * 8);
    const i32x4 rml = buffer_rsrc(mlb, rng);
    const uint32_t mdst = (uint32_t)(uintptr_t)(char LDS_AS*)mlt;
    for (int i = 0; i < nml; ++i) {
      const int e = 64 * i + lane;  // entry index: (j G + sp) 2 + f
      const int j = e >> (gsh + 1), sp = (e >> 1) & (G - 1), f = e & 1;
      const uint32_t off = (sp < S && j < RPW) ? (uint32_t)(sp * sstride * 8 + j * a.H * 8 + 4 * f) : 0xfffffff0u;
      dma4(rml, mdst + 256u * (uint32_t)i, off);
    }
  }
  gather(0);
  const int ps0 = pass_splits(0);
  const int g0 = n > 0 ? ps0 * n : 0;  // partial-row loads of the first pass
  wait_vm_le(g0);

  const size_t wrow = ((size_t)h * kRowsPerHead + kNope + 32 * wave + (lane & 31)) * kLatent + 8 * hh;
  const uint16_t* w = a.wkv_b + wrow;
  const uint8_t* w8 = a.fp8.w_fp8 + wrow;
  bf16x8 wf[32];
  uint2 wr[FP8 ? 32 : 1];
  auto load_w = [&](int st) __attribute__((always_inline)) {
    if constexpr (FP8) wr[st] = *reinterpret_cast<const uint2*>(w8 + 16 * st);
    else wf[st] = ld8(w + 16 * st);
  };

  // Merge weights g_s = 2^(m_s - M) / L of the row, from a group max and a
  // group sum over the row's G lanes, into a per-wave table (an all -inf row
  // gets NaN weights: an empty selection, as in mla_combine).  In pass q lane
  // l takes row j = q R + l / G and split s = l % G: table entries 64 q + l.
  float* wt = reinterpret_cast<float*>(wtab) + wave * RPW * 64;
  if constexpr (FUSED) {
    constexpr int kMaxPasses = RPW;  // G = 64
#pragma unroll
    for (int q = 0; q < kMaxPasses; ++q) {
      if (q * R >= RPW) continue;
      const int j = q * R + (lane >> gsh), sp = lane & (G - 1);
      const float2 ml = (j < RPW && sp < S) ? mlt[64 * q + lane] : float2{-INFINITY, 0.f};
      float M = ml.x;
      for (int o = 1; o < G; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
      const float e = (ml.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
      float L = e * ml.y;
      for (int o = 1; o < G; o <<= 1) L += __shfl_xor(L, o);
      if (j < RPW && sp < S) wt[j * 64 + sp] = L > 0.f ? e / L : __builtin_nanf("");
      if (j < RPW && sp == 0 && r0 + j < nrows) {
        const int64_t bh = (int64_t)(b0 + r0 + j) * a.H + h;
        if (a.lse != nullptr) a.lse[bh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
        if (a.status != nullptr && h == 0 && !(L > 0.f)) atomicOr(a.status, 4u);
      }
    }
  }
  float v[RPW][8];
#pragma unroll
  for (int j = 0; j < RPW; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) v[j][k] = 0.f;

  // Merge step: split c0 + c of the pass, row j.
  auto merge_step = [&](int c0, int c, int j) __attribute__((always_inline)) {
    const float gs = FUSED ? wt[j * 64 + c0 + c] : 1.f;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(slots + slot_of(c * n + j) * kOtRow + 16 * lane);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[j][k] += gs * (float)x[k];
  };
  if (n == RPW) {
    // A full wave.  First pass: split sc's rows are the oldest loads left
    // once (ps0 - 1 - sc) RPW partial loads and the W_UV,h loads issued so
    // far are outstanding; the W_UV,h loads ride beside the merge steps,
    // 32 / (SPP RPW) per step (those of steps past the pass still go out).
    constexpr int kLoadsPerStep = 32 / (SPP * RPW);
#pragma unroll
    for (int sc = 0; sc < SPP; ++sc) {
      if (sc < ps0) wait_vm_le((ps0 - 1 - sc) * RPW + sc * RPW * kLoadsPerStep);
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
#pragma unroll
        for (int u = 0; u < kLoadsPerStep; ++u) {
          const int st = (sc * RPW + j) * kLoadsPerStep + u;
          load_w(st);
        }
        if (sc < ps0) merge_step(0, sc, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    for (int c0 = SPP; c0 < S; c0 += SPP) {
      // The previous pass's slot reads must be complete before its slots are
      // gathered into again.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      gather(c0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const int ps = pass_splits(c0);
#pragma unroll
      for (int sc = 0; sc < SPP; ++sc) {
        if (sc >= ps) break;
#pragma unroll
        for (int j = 0; j < RPW; ++j) merge_step(c0, sc, j);
      }
    }
  } else {
    // A wave with fewer rows (or none): W_UV,h at once, then passes of
    // kCap / n splits.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int st = 0; st < 32; ++st) load_w(st);
    if (n > 0) {
      for (int c0 = 0; c0 < S;) {
        const int ps = pass_splits(c0);
        if (c0 > 0) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          gather(c0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        for (int c = 0; c < ps; ++c)
#pragma unroll
          for (int j = 0; j < RPW; ++j)
            if (j < n) merge_step(c0, c, j);
        c0 += ps;
      }
    }
  }
  // Merged rows (bf16) into the split-0 slots; every wave's rows must be
  // there before the products read the whole tile.
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    bf16x8 y;
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = (__bf16)v[j][k];
    *reinterpret_cast<bf16x8*>(slots + (r0 + j) * kOtRow + 16 * lane) = y;
  }
  __syncthreads();

  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (__builtin_expect(wtie[j], 0)) {
#pragma unroll
        for (int st = 8 * j; st < 8 * j + 8; ++st) wf[st] = dq8<true>(wr[st], wsc[j]);
      } else {
#pragma unroll
        for (int st = 8 * j; st < 8 * j + 8; ++st) wf[st] = dq8<false>(wr[st], wsc[j]);
      }
    }
    if (a.fp8.w_formed != nullptr && b0 == 0) {
#pragma unroll
      for (int st = 0; st < 32; ++st) *reinterpret_cast<bf16x8*>(a.fp8.w_formed + wrow + 16 * st) = wf[st];
    }
  }
  // N = 32 tile rows; with ROWS = 16 the upper 16 columns are not written.
  f32x16 acc = {};
  const char LDS_AS* ol = (const char LDS_AS*)slots + (lane & 31) * kOtRow + 16 * hh;
#pragma unroll
  for (int st = 0; st < 32; ++st) acc = mfma32(wf[st], *(const bf16x8 LDS_AS*)(ol + 32 * st), acc);
  const int r = lane & 31;
  if (r < nrows) {
    uint16_t* out = a.out + (int64_t)(b0 + r) * a.out_sb + (int64_t)h * a.out_sh + 32 * wave + 4 * hh;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<uint2*>(out + 8 * q4) = pack4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
  }
}

// ---------------------------------------------------------------------------
// value-up of merged rows at large batches (o_latent given, e.g. the prefill's
// B * T rows): workgroup = (head, slice of the batch's 32-row tiles), the
// slices of a head on one XCD.  W_UV,h is formed in registers once per
// workgroup (value_up_kernel forms it once per tile, so at thousands of rows
// every tile re-read it); the slice's tiles stream through four LDS buffers,
// wave w moving rows 8 w .. 8 w + 7 of each (one 1 KB row per LDS-DMA
// instruction, rows past B masked), three tiles ahead, one barrier per tile.
// Each tile is multiplied exactly as in value_up_kernel (same operands, same
// order): the results are identical.
// ---------------------------------------------------------------------------
constexpr int kVsNbuf = 4;
template <bool FP8>
__global__ __launch_bounds__(256, 1) void value_up_stream_kernel(const ValueUpArgs a, int groups) {
  __shared__ __attribute__((aligned(1024))) char tiles[kVsNbuf * 32 * kOtRow];
  const int units = a.H * groups;
  const int per_xcd = (units + 7) >> 3;
  const int unit = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (unit >= units) return;
  const int h = unit / groups, g = unit % groups;
  const int ntiles = (a.B + 31) / 32;
  const int t0 = (int)((int64_t)ntiles * g / groups), t1 = (int)((int64_t)ntiles * (g + 1) / groups);
  if (t0 >= t1) return;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(char LDS_AS*)tiles;
  const uint32_t row_bytes = (uint32_t)a.H * kLatent * 2u;  // between consecutive batch rows of one head

  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t buf = lds0 + (uint32_t)((t % kVsNbuf) * 32 * kOtRow);
    const int nv = t < t1 ? min(32, a.B - 32 * t) : 0;  // rows of the tile that exist (none past the slice)
    const i32x4 rs = buffer_rsrc(a.o_latent + ((int64_t)(t < t1 ? 32 * t : 0) * a.H + h) * kLatent,
                                 nv > 0 ? (uint32_t)(nv - 1) * row_bytes + 1024u : 0u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t r = (uint32_t)(8 * wave + j);
      dma16(rs, buf + r * (uint32_t)kOtRow, r * row_bytes + 16u * (uint32_t)lane);
    }
  };
  issue(t0);
  issue(t0 + 1);
  issue(t0 + 2);

  // W_UV,h rows 32 w + l % 32, columns 16 st + 8 (l / 32) .. + 7, as in
  // value_up_kernel.  Pinned before the loop: the compiler's wait for these
  // loads (which also covers the three tiles issued before them) sits here,
  // and none inside the loop drains the tiles in flight.
  const size_t wrow = ((size_t)h * kRowsPerHead + kNope + 32 * wave + (lane & 31)) * kLatent + 8 * hh;
  bf16x8 wf[32];
  if constexpr (FP8) {
    uint2 wr[32];
#pragma unroll
    for (int st = 0; st < 32; ++st) wr[st] = *reinterpret_cast<const uint2*>(a.fp8.w_fp8 + wrow + 16 * st);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = a.fp8.w_scale[(2 * h + 1) * (kLatent / 128) + j];
      if (__builtin_expect(block_has_ties(sc, lane), 0)) {
#pragma unroll
        for (int st = 8 * j; st < 8 * j + 8; ++st) wf[st] = dq8<true>(wr[st], sc);
      } else {
#pragma unroll
        for (int st = 8 * j; st < 8 * j + 8; ++st) wf[st] = dq8<false>(wr[st], sc);
      }
    }
    if (a.fp8.w_formed != nullptr && t0 == 0) {
#pragma unroll
      for (int st = 0; st < 32; ++st) *reinterpret_cast<bf16x8*>(a.fp8.w_formed + wrow + 16 * st) = wf[st];
    }
  } else {
#pragma unroll
    for (int st = 0; st < 32; ++st) wf[st] = ld8(a.wkv_b + wrow + 16 * st);
  }
#pragma unroll
  for (int st = 0; st < 32; ++st) asm volatile("" : "+v"(wf[st]));

  for (int t = t0; t < t1; ++t) {
    // This wave's rows of tile t are in when at most 16 of its memory
    // operations are outstanding: tiles t + 1 and t + 2 are 16 loads, and
    // the output stores of the iterations since also count, so the wait is
    // conservative (it can cover part of tile t + 1, never end early).  The
    // barrier makes the tile every wave's and frees buffer (t + 3) % 4, read
    // in the previous iteration.
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    __syncthreads();
    issue(t + 3);
    f32x16 acc = {};
    const char LDS_AS* ol = (const char LDS_AS*)tiles + (t % kVsNbuf) * 32 * kOtRow + (lane & 31) * kOtRow + 16 * hh;
#pragma unroll
    for (int st = 0; st < 32; ++st) acc = mfma32(wf[st], *(const bf16x8 LDS_AS*)(ol + 32 * st), acc);
    const int b = 32 * t + (lane & 31);
    if (b < a.B) {
      uint16_t* out = a.out + (int64_t)b * a.out_sb + (int64_t)h * a.out_sh + 32 * wave + 4 * hh;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<uint2*>(out + 8 * q4) = pack4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
    }
  }
  // The masked loads issued past the slice may still be landing.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// decode: sparse flash-decode over the selected cache rows.
//
// Workgroup = (sequence b, key split s), all 128 heads, 4 waves, one
// workgroup per CU.  Keys are processed in blocks of 32.  Each block of rows
// is gathered into LDS by buffer loads that write LDS directly (16 bytes per
// lane; 8 adjacent lanes read one whole 128-byte line of one row); masked
// slots get an offset past the record range, so their rows arrive as zeros.
//
// LDS block layout: a row [latent 512 | rotary 64] is 9 lines of 128 bytes
// (8 chunks of 8 features).  Line m of key k is the segment (m * 32 + k) * 128
// and chunk q of that line sits at 16-byte position q ^ sw(k); sw() keeps the
// score reads (32 keys, one chunk) and the transpose reads (4 keys x 4
// chunks per 16 lanes) on distinct banks.
//
// Wave w owns heads 32 w .. 32 w + 31 through the whole block:
//   scores  S^T[key][head] = sum_f row[key][f] Q~[head][f]; A = rows (LDS,
//           ds_read_b128), B = [q~ | q_pe] of the wave's heads held in
//           registers; M = keys, N = heads; one dependent chain of 36 MFMAs.
//   softmax each lane holds 16 keys of one head (lanes l and l ^ 32 share a
//           head): in-lane max and sum plus one lane swap; exp2 with
//           scale * log2 e folded in; lazy rescaling (the reference maximum
//           moves only when a block exceeds it by 2^8).
//   mix     O~^T[col][head] += sum_key C^T[col][key] P^T[key][head] over all
//           512 columns; A = C^T through transpose reads, B = P straight from
//           the softmax registers (the keys permuted alike in A and B);
//           M = columns, N = heads, K = keys; 32 MFMAs.
// P, the rescale decision and the running (max, sum) never leave the wave:
// the only dependency between waves is the gathered block itself.
//
// Software pipeline, iteration j, after one barrier (block j has landed):
//   A  the score chain of block j: 36 dependent MFMAs and their operand
//      reads, nothing else (any other work there holds back the next MFMA);
//   B  the mix of block j - 1: 32 independent MFMAs, with the softmax of
//      block j spread over their slots and the gather of block j + 2 going
//      out one line every third slot.
// Four row buffers: j - 1 (mix), j (scores), j + 1 and j + 2 (in flight).
// Buffer (j + 2) % 4 last held block j - 2, mixed in iteration j - 1, which
// every wave has finished before the barrier of iteration j.  Gathers past
// the last block load masked rows (zeros) into their buffer, so exactly one
// block (9 loads per wave) is always in flight behind the one waited for.
// ---------------------------------------------------------------------------
constexpr int kBlk = 32;                    // keys per block
constexpr int kNbuf = 4;                    // row buffers
constexpr int kBufBytes = 72 * kBlk * 16;   // 36864: one block of rows
// Query staging in the prologue: lines 7 and 8 of each wave's 32 head rows
// in buffer 0 (8 KB per wave), lines 0 .. 6 from buffer 1 on (28 KB per
// wave, 4 KB past buffer 3), so that block 0 can be gathered into buffer 0
// while the bulk of the query is still arriving.
constexpr int kOffQ = kBufBytes;
constexpr int kQWave = 7 * kBlk * 128;
constexpr int kOffIdx = kOffQ + 4 * kQWave;  // int [kIdxCap]
constexpr int kOffLen = kOffIdx + kIdxCap * 4;  // int [4][64]: the sequence length, per wave
constexpr int kOffTot = kOffLen + 4 * 64 * 4;   // int [2][4]: valid slots per half and wave (compaction)
constexpr int kDecodeLds = kOffTot + 8 * 4;
constexpr int kSoftSteps = 32;              // softmax steps placed beside MFMAs
static_assert(kDecodeLds <= 160 * 1024, "decode LDS budget");
constexpr int kTilePitch = 1040;            // output tile row: 512 bf16 + 16 bytes of padding
static_assert(kHeads * kTilePitch <= kNbuf * kBufBytes, "the epilogue tile must stay inside the row buffers");
static_assert(kOffIdx >= kNbuf * kBufBytes, "the index list must not overlap the row buffers");
static_assert(kSoftSteps <= 32, "the softmax steps must fit the slots of a mix");

template <bool DENSE, bool SPLIT>
__global__ __launch_bounds__(256, 1) void decode_kernel(const DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kDecodeLds];
  char LDS_AS* s3 = (char LDS_AS*)smem;
  int* sidx = reinterpret_cast<int*>(smem + kOffIdx);

  // Units (row, split) are numbered so that the splits of a row run on one
  // XCD (workgroup x is dispatched to XCD x % 8): the row's query tile then
  // comes from HBM once and from that XCD's L2 after.
  // Prefill: row b is query token b % T of prompt b / T, whose keys are the
  // prompt's own positions (one cache per prompt), causally limited to the
  // token's own position.  Decode: row b is sequence b.
  const bool causal = a.causal != 0;
  int b, s;
  if (!causal) {
    // Each XCD takes a contiguous range of units.
    const int units = a.B * a.S;
    const int per_xcd = (units + 7) >> 3;
    const int unit = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (unit >= units) return;
    b = unit / a.S;
    s = unit % a.S;
  } else {
    // A token's work grows with its position (its masked slots cost no
    // blocks), so rows are dealt to the XCDs in turn, latest tokens first:
    // every XCD gets an even share and the longest workgroups start first.
    // Dispatch-order row j (the XCD's (i / S)-th, i its workgroup count on
    // that XCD) is token T - 1 - j / P of prompt j % P (P prompts).
    const int j = (int)(blockIdx.x >> 3) / a.S * 8 + (int)(blockIdx.x & 7);
    if (j >= a.B) return;
    const int T = a.rows_per_seq, P = a.B / a.rows_per_seq;
    b = (j % P) * T + (T - 1 - j / P);
    s = (int)(blockIdx.x >> 3) % a.S;
  }
  const int seq = causal ? b / a.rows_per_seq : b;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int head = 32 * wave + (lane & 31);   // this lane's head throughout

  constexpr bool dense = DENSE;
  const bool validate = (a.flags & 1u) != 0;
  const int s0 = s * a.chunk;
  const int s1 = min(a.k_max, s0 + a.chunk);
  const int nslot = max(0, s1 - s0);
  // Slots actually walked, decided once the length and the index list are in
  // (below): unless the scores of every slot are requested, the valid slots
  // of an index list are moved to its front and a dense split stops at L_b,
  // so masked slots cost no blocks.
  int nkeys = nslot;

  const uint32_t lds0 = (uint32_t)(uintptr_t)s3;
  // Score-read offsets: row lane % 32 of a tile laid out like a gathered
  // block, chunk 2 st + hh of line st / 4.
  uint32_t qk_base[4];
  {
    const uint32_t key = (uint32_t)(lane & 31);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      qk_base[s4] = key * 128u + (((uint32_t)(2 * s4 + hh)) ^ seg_swz(key)) * 16u;
  }

  // Query operand [q~ (512) | q_pe (64)] for this lane's head, in MFMA B
  // layout.  Read straight from HBM, each load would touch 32 rows for 32
  // bytes apiece; instead each wave moves its 32 heads' rows into LDS with
  // whole-line LDS-DMA (8 lanes per 128-byte line, lines laid out and
  // swizzled like those of a gathered block: head row r as key r) and reads
  // the operand back with the score reads.  The B layout (n = lane % 32,
  // k = 8 (lane / 32) + v) is the A layout of the score operand, so the same
  // reads serve.  Lines 7 and 8 go to buffer 0, lines 0 .. 6 to the region
  // at kOffQ; line m of the tile at `base` + m * 4 KB either way.
  bf16x8 qf[36];
  auto query_base = [&](int m) __attribute__((always_inline)) -> uint32_t {
    return m >= 7 ? (uint32_t)(8192 * wave + (m - 7) * kBlk * 128)
                  : (uint32_t)(kOffQ + kQWave * wave + m * kBlk * 128);
  };
  auto stage_query = [&](int m0, int m1) __attribute__((always_inline)) {
    // Heads past a.H (a head-sharded call) lie past both ranges and load zeros.
    const i32x4 rq = buffer_rsrc(a.q_abs + (int64_t)b * a.H * kLatent, (uint32_t)(a.H * kLatent * 2));
    const i32x4 rp = buffer_rsrc(a.q_pe + (int64_t)b * a.q_pe_sb,
                                 (uint32_t)(((int64_t)(a.H - 1) * a.q_pe_sh + kRope) * 2));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t r = (uint32_t)(8 * g + (lane >> 3));
      const uint32_t q16 = (((uint32_t)(lane & 7)) ^ seg_swz(r)) * 16u;
      const uint32_t hrow = (uint32_t)(32 * wave) + r;
#pragma unroll
      for (int m = m0; m < m1; ++m) {
        const uint32_t dst = lds0 + query_base(m) + (uint32_t)(8 * g * 128);
        if (m < 8) dma16(rq, dst, hrow * (uint32_t)(kLatent * 2) + (uint32_t)(m * 128) + q16);
        else dma16(rp, dst, hrow * (uint32_t)(a.q_pe_sh * 2) + q16);
      }
    }
  };
  auto read_query = [&](int st0, int st1) __attribute__((always_inline)) {
#pragma unroll
    for (int st = st0; st < st1; ++st)
      qf[st] = *(const bf16x8 LDS_AS*)(s3 + query_base(st >> 2) + qk_base[st & 3]);
  };

  // Every load of the prologue is an LDS-DMA: query lines 7 and 8 (8 per
  // wave), the sequence length (lane 0 of each wave; the other lanes read
  // past the 4-byte range and land zeros), this split's index slots (slot i
  // lands at sidx[i], in groups of 256; slots past nslot are masked below),
  // then query lines 0 .. 6 (28 per wave).  With no
  // compiler-visible load the only waits are the explicit ones below (a
  // compiler-placed wait for an ordinary load would also drain the query
  // rows; a scalar load of the length would be waited on with the kernel
  // arguments, before anything else goes out).
  stage_query(7, 9);
  // (In prefill mode there is no length array: a zero-byte range loads zeros.)
  dma4(causal ? buffer_rsrc(a.q_abs, 0u) : buffer_rsrc(a.seq_lens + b, 4u),
       lds0 + (uint32_t)(kOffLen + 256 * wave), 4u * (uint32_t)lane);
  if constexpr (!dense) {
    // 4 bytes per lane, so that the range check (nslot slots) is per slot.
    // Wave w moves the slots its own threads validate below (each wave waits
    // for its own loads only): 256 w .. 256 w + 255, and with more than 1024
    // slots also 1024 + 256 w .. 1024 + 256 w + 255.
    const i32x4 ri = buffer_rsrc(a.indices + (int64_t)b * a.k_max + s0, (uint32_t)nslot * 4u);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      dma4(ri, lds0 + (uint32_t)(kOffIdx + 4 * (256 * wave + 64 * k)), 4u * (uint32_t)(256 * wave + 64 * k + lane));
    if (nslot > kIdxCap / 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        dma4(ri, lds0 + (uint32_t)(kOffIdx + 4 * (kIdxCap / 2 + 256 * wave + 64 * k)),
             4u * (uint32_t)(kIdxCap / 2 + 256 * wave + 64 * k + lane));
    }
  }
  stage_query(0, 7);
  asm volatile("s_waitcnt vmcnt(28)" ::: "memory");
  read_query(28, 36);
  const int Lb = causal ? min(b % a.rows_per_seq + 1, a.max_len)
                        : __builtin_amdgcn_readfirstlane(
                              min(max(*(const volatile int LDS_AS*)(s3 + kOffLen + 256 * wave), 0), a.max_len));

  // Stage this split's index slots as cache rows (-1 = masked).  The same
  // predicate decides validity, the attended bitmap and the device checks.
  const bool keep_slots = (a.flags & 2u) != 0;  // per-slot scores: slot order kept
  if constexpr (!dense) {
    {
      // Thread tid: slots 4 tid .. 4 tid + 3 of each half (h = 0: slot
      // 4 tid + e, h = 1: slot 1024 + 4 tid + e; past nslot: masked).
      int r[2][4];
      int cnt[2] = {0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i0 = h * (kIdxCap / 2) + 4 * tid;
        const int4 raw = *reinterpret_cast<const int4*>(sidx + i0);
        const int v[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = v[e];
          const bool ok = (i0 + e < nslot) && t >= 0 && t < Lb;
          if (validate && i0 + e < nslot) {
            // Prefill: a key after the token (but inside the prompt) is
            // removed by the causal mask, not an error.
            if (!ok && t != -1 && !(causal && t >= Lb && t < a.max_len)) atomicOr(a.status, 1u);
            if (ok) {
              const uint32_t bit = 1u << (t & 31);
              const uint32_t old = atomicOr(a.bitmap + (int64_t)b * a.bitmap_words + (t >> 5), bit);
              if (old & bit) atomicOr(a.status, 2u);
            }
          }
          r[h][e] = ok ? t : -1;
          cnt[h] += ok ? 1 : 0;
        }
      }
      if (keep_slots) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *reinterpret_cast<int4*>(sidx + h * (kIdxCap / 2) + 4 * tid) = make_int4(r[h][0], r[h][1], r[h][2], r[h][3]);
      } else {
        // Stable compaction: the valid slots, in slot order, to the front.
        // A slot's place = the valid slots before it: in its half, those of
        // the threads before this one (within the wave from the three bit
        // planes of the count, 0 .. 4; across waves from per-wave totals in
        // LDS), after all of the first half's for the second.
        auto below = [&](uint64_t m) __attribute__((always_inline)) {
          return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        };
        int* stot = reinterpret_cast<int*>(smem + kOffTot);  // [half][wave]
        int before[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint64_t p0 = __builtin_amdgcn_ballot_w64((cnt[h] & 1) != 0);
          const uint64_t p1 = __builtin_amdgcn_ballot_w64((cnt[h] & 2) != 0);
          const uint64_t p2 = __builtin_amdgcn_ballot_w64((cnt[h] & 4) != 0);
          before[h] = below(p0) + 2 * below(p1) + 4 * below(p2);
          if (lane == 0) stot[4 * h + wave] = __popcll(p0) + 2 * __popcll(p1) + 4 * __popcll(p2);
        }
        __syncthreads();  // the totals are in; every thread holds its raw slots
        int base[2] = {0, 0}, total = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          base[h] = total;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int tw = stot[4 * h + w];
            base[h] += w < wave ? tw : 0;
            total += tw;
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int pos = base[h] + before[h];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (r[h][e] >= 0) sidx[pos++] = r[h][e];
        }
        // The last block's slots past the valid ones are masked.
        for (int i = total + tid; i < ((total + kBlk - 1) & ~(kBlk - 1)); i += 256) sidx[i] = -1;
        nkeys = total;
      }
    }
  } else {
    if (validate) {
      for (int i = tid; i < nslot; i += 256) {
        const int t = s0 + i;
        if (t < Lb) atomicOr(a.bitmap + (int64_t)b * a.bitmap_words + (t >> 5), 1u << (t & 31));
      }
    }
    // Positions from L_b on are masked: the split stops there.
    if (!keep_slots) nkeys = max(0, min(nslot, Lb - s0));
  }
  const int nblk = __builtin_amdgcn_readfirstlane((nkeys + kBlk - 1) / kBlk);
  // Every wave has read its query lines 7 and 8 out of buffer 0 before this
  // barrier, after which block 0 is gathered there.
#pragma unroll
  for (int st = 28; st < 36; ++st) asm volatile("" : "+v"(qf[st]));
  __syncthreads();

  uint16_t* dst = !SPLIT ? a.o_latent + (int64_t)b * a.H * kLatent
                             : a.part_o + ((int64_t)s * a.B + b) * a.H * kLatent;
  if (nblk == 0) {
    // The query rows may still be landing in this workgroup's LDS.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // No slot in this split: the normalised mix is NaN with S == 1 (an empty
    // selection); with several splits the (unnormalised) sum is 0 and the
    // merge gives it no weight.  (max, sum) = (-inf, 0).  Everything below
    // may then assume a block.
    const uint32_t fb = !SPLIT ? 0x7fc07fc0u : 0u;
    for (int i = tid; i < a.H * kLatent / 8; i += 256)
      reinterpret_cast<uint4*>(dst)[i] = uint4{fb, fb, fb, fb};
    if (tid < a.H) {
      if constexpr (!SPLIT) {
        if (a.lse != nullptr) a.lse[(int64_t)b * a.H + tid] = -INFINITY;
        if (validate && tid == 0) atomicOr(a.status, 4u);
      } else {
        float* pml = a.part_ml + (((int64_t)s * a.B + b) * a.H + tid) * 2;
        pml[0] = -INFINITY;
        pml[1] = 0.f;
      }
    }
    return;
  }

  auto row_of = [&](int i) __attribute__((always_inline)) -> int {  // slot i of this split -> cache row or -1
    if constexpr (dense) {
      const int t = s0 + i;
      return (i < nslot && t < Lb) ? t : -1;
    }
    return sidx[i];
  };

  const uint32_t kv_rb = (uint32_t)(a.kv_st * 2), pe_rb = (uint32_t)(a.pe_st * 2);
  const i32x4 rkv = buffer_rsrc(a.kv + (int64_t)seq * a.kv_sb, (uint32_t)Lb * kv_rb);
  const i32x4 rpe = buffer_rsrc(a.pe + (int64_t)seq * a.pe_sb, (uint32_t)Lb * pe_rb);
  // Gather block p into buffer p % 4: wave w moves keys 8 w .. 8 w + 7, all
  // 9 lines; lane l takes key 8 w + l / 8 and 16-byte position l % 8.
  struct Gather {
    uint32_t okv, ope, dst;
  };
  auto gather_setup = [&](int p) __attribute__((always_inline)) {
    const int key = 8 * wave + (lane >> 3);
    const int row = p < nblk ? row_of(p * kBlk + key) : -1;
    const uint32_t q16 = (((uint32_t)(lane & 7)) ^ seg_swz((uint32_t)key)) * 16u;
    Gather g;
    g.okv = row >= 0 ? (uint32_t)row * kv_rb + q16 : kMaskedOffset;
    g.ope = row >= 0 ? (uint32_t)row * pe_rb + q16 : kMaskedOffset;
    g.dst = lds0 + (uint32_t)((p % kNbuf) * kBufBytes) + (uint32_t)(8 * wave) * 128u;
    return g;
  };
  // Line m (0..7 latent, 8 rotary) of a block's gather.
  auto gather_line = [&](const Gather& g, int m) __attribute__((always_inline)) {
    if (m < 8) dma16(rkv, g.dst + (uint32_t)(m * kBlk * 128), g.okv + (uint32_t)(m * 128));
    else dma16(rpe, g.dst + (uint32_t)(8 * kBlk * 128), g.ope);
  };
  auto issue = [&](int p) __attribute__((always_inline)) {
    const Gather g = gather_setup(p);
#pragma unroll
    for (int m = 0; m < 9; ++m) gather_line(g, m);
  };

  // Transpose-read offsets (mix A operand, column tile mt, k-step ks): in
  // each 16-lane group (gm = group & 1) source lane i reads key
  // 16 ks + 8 r + 4 hh + i / 4 for the fragment's two reads r = 0, 1, and
  // columns 32 mt + 16 gm + 4 (i % 4) .. + 3: line mt / 2, chunk
  // 4 (mt % 2) + 2 gm + (i % 4) / 2, byte 8 (i % 2).  Output lane l then holds
  // column 32 mt + l % 32 with key 16 ks + 8 r + 4 hh + e at k = 8 hh + 4 r + e,
  // which is where the score layout leaves that key's P: the score
  // accumulator element 8 ks + 4 r + e of lane l is key 16 ks + 8 r + 4 hh + e.
  const int i16 = lane & 15, gm = (lane >> 4) & 1;
  uint32_t pc_base[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1) {
      const uint32_t key = (uint32_t)(8 * r + 4 * hh + (i16 >> 2));
      const uint32_t q = (uint32_t)(4 * c1 + 2 * gm + ((i16 & 3) >> 1));
      pc_base[r][c1] = key * 128u + ((q ^ seg_swz(key)) * 16u) + 8u * (uint32_t)(i16 & 1);
    }

  // acc[mt][v]: column 32 mt + 8 (v / 4) + 4 hh + v % 4, head `head`.
  f32x16 acc[16];
#pragma unroll
  for (int mt = 0; mt < 16; ++mt) acc[mt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // acc *= alpha (this lane's head) on the accumulator registers in place (a
  // C++ multiply would move all 256 accumulators into vector registers).
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float tmp;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(acc[mt][v]), "=&v"(tmp)
                     : "v"(alpha));
      }
    asm volatile("s_nop 3" ::: "memory");
  };

  // Key-validity ballot of block j: bit k of the result = slot j * 32 + k
  // holds a row.
  auto valid_mask = [&](int j) __attribute__((always_inline)) -> uint32_t {
    const bool v_ok = row_of(j * kBlk + (lane & 31)) >= 0;
    return (uint32_t)__builtin_amdgcn_ballot_w64(v_ok);
  };
  // x[v] is key 8 (v / 4) + 4 hh + v % 4 of the block.
  auto key_ok = [&](uint32_t vmj, int v) __attribute__((always_inline)) -> bool {
    return ((vmj >> (8 * (v >> 2) + 4 * hh + (v & 3))) & 1u) != 0;
  };
  // Raw scores of block j (scale applied, -inf where masked).
  auto write_scores = [&](int j, const f32x16& x, uint32_t vmj) __attribute__((always_inline)) {
    if (head >= a.H) return;
    float* so = a.scores + ((int64_t)b * a.H + head) * a.k_max + s0 + j * kBlk;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kloc = 8 * (v >> 2) + 4 * hh + (v & 3);
      if (j * kBlk + kloc < nslot) so[kloc] = key_ok(vmj, v) ? x[v] * a.scale : -INFINITY;
    }
  };
  // Before the softmax of a block: a block with masked keys is scaled here
  // (-inf where masked) and its softmax factor becomes 1.
  auto prepare = [&](f32x16& x, uint32_t vmj) __attribute__((always_inline)) -> float {
    if (vmj == 0xffffffffu) return a.scale_log2;
#pragma unroll
    for (int v = 0; v < 16; ++v) x[v] = key_ok(vmj, v) ? x[v] * a.scale_log2 : -INFINITY;
    return 1.f;
  };

  // Softmax of the block in x (this lane's 16 scores; cx takes them to log2
  // units), in steps 0 .. kSoftSteps - 1 of a few vector instructions each,
  // so that each fits the issue slot beside one MFMA.  Leaves P in pb, the
  // factor alpha for the accumulators and the wave-uniform decision resc_any
  // to apply it.  Each step's results are pinned where they are computed;
  // otherwise the compiler sinks the vector work to its uses in the mix.
  float mloc = 0.f, mblk = 0.f, alpha = 1.f, mref = 0.f, lsum = 0.f;
  bool resc = false, resc_any = false;
  uint32_t pk[8];  // P as bf16 pairs, keys in the order of x
  auto soft_step = [&](int k, f32x16& x, float cx, bf16x8 (&pb)[2]) __attribute__((always_inline)) {
    if (k < 8) {  // scale two scores, running max
      x[2 * k] *= cx;
      x[2 * k + 1] *= cx;
      const float m2 = fmaxf(x[2 * k], x[2 * k + 1]);
      mloc = (k == 0) ? m2 : fmaxf(mloc, m2);
      asm volatile("" : "+v"(x[2 * k]), "+v"(x[2 * k + 1]), "+v"(mloc));
    } else if (k == 8) {  // the other half of this head's keys sits in lane l ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
      mblk = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      asm volatile("" : "+v"(mblk));
    } else if (k == 9) {
      // Move the reference max when this block exceeds it by more than 2^8;
      // a head's accumulators are still zero while its max is -inf.
      const bool need = mblk > m_run + kRescaleLog2;
      resc = need && m_run != -INFINITY;
      const float mnew = need ? mblk : m_run;
      alpha = resc ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.f;
      mref = (mnew == -INFINITY) ? 0.f : mnew;
      m_run = mnew;
      asm volatile("" : "+v"(alpha), "+v"(m_run), "+v"(mref));
    } else if (k == 10) {
      l_run *= alpha;
      resc_any = __builtin_amdgcn_ballot_w64(resc) != 0;
      asm volatile("" : "+v"(l_run));
    } else if (k < 27) {  // one probability per step
      const int v = k - 11;
      x[v] = __builtin_amdgcn_exp2f(x[v] - mref);
      lsum = (v == 0) ? x[v] : lsum + x[v];
      asm volatile("" : "+v"(x[v]), "+v"(lsum));
    } else if (k < 31) {  // pack P, four probabilities per step
      const int q = 2 * (k - 27);
      pk[q] = pack2(x[2 * q], x[2 * q + 1]);
      pk[q + 1] = pack2(x[2 * q + 2], x[2 * q + 3]);
      asm volatile("" : "+v"(pk[q]), "+v"(pk[q + 1]));
    } else {
      pb[0] = __builtin_bit_cast(bf16x8, uint4{pk[0], pk[1], pk[2], pk[3]});
      pb[1] = __builtin_bit_cast(bf16x8, uint4{pk[4], pk[5], pk[6], pk[7]});
      l_run += lsum;
      asm volatile("" : "+v"(l_run));
    }
  };

  // Mix of block p (rows in buffer p % 4) with this wave's P fragments pb[ks]:
  // fragment i = 16 ks + mt, one MFMA each, A fragments read four ahead.
  // With SOFT, the softmax steps of the next block (x -> pn) ride beside the
  // MFMAs, one per MFMA, and the gather `gn` goes out one line every third
  // slot (a burst of gathers from four waves backs up the CU's address unit).
  // The mix MFMAs are independent of each other, so this work delays none.
  auto mix = [&](auto soft_tag, int p, const bf16x8 (&pb)[2], f32x16& x, float cx,
                 bf16x8 (&pn)[2], const Gather* gn) __attribute__((always_inline)) {
    constexpr bool SOFT = decltype(soft_tag)::value;
    const char LDS_AS* buf = s3 + (p % kNbuf) * kBufBytes;
    auto av_ld = [&](int i) {
      const int ks = i >> 4, mt = i & 15;
      const uint32_t o = (uint32_t)((mt >> 1) * kBlk * 128 + ks * 16 * 128);
      return tr_pair(buf + pc_base[0][mt & 1] + o, buf + pc_base[1][mt & 1] + o);
    };
    constexpr int MA = 4;
    bf16x8 ring[MA + 1];
#pragma unroll
    for (int i = 0; i < MA; ++i) ring[i] = av_ld(i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + MA < 32) ring[(i + MA) % (MA + 1)] = av_ld(i + MA);
      acc[i & 15] = mfma32(ring[i % (MA + 1)], pb[i >> 4], acc[i & 15]);
      if (SOFT && i < kSoftSteps) soft_step(i, x, cx, pn);
      if (SOFT && i % 3 == 1 && i / 3 < 9) gather_line(*gn, i / 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Score chain of block j into sacc: 36 MFMAs, each depending on the one
  // before, so nothing but the operand reads sits between them (other work
  // there would hold back the next MFMA of the chain).  With `gn`, that
  // gather goes out one line every fourth slot (block 0 only).  Every score
  // operand is read three slots ahead; a ring slot is reloaded after the MFMA
  // that follows its last use has issued.
  auto chain = [&](int j, f32x16& sacc, const Gather* gn) __attribute__((always_inline)) {
    const char LDS_AS* kbuf = s3 + (j % kNbuf) * kBufBytes;
    constexpr int AH = 3;
    bf16x8 ring[AH + 1];
    auto qk_ld = [&](int st) {
      return *(const bf16x8 LDS_AS*)(kbuf + qk_base[st & 3] + (uint32_t)((st >> 2) * kBlk * 128));
    };
#pragma unroll
    for (int st = 0; st < AH; ++st) ring[st] = qk_ld(st);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 36; ++k) {
      if (gn != nullptr && (k & 3) == 0) gather_line(*gn, k >> 2);
      const bf16x8 kf = ring[k % (AH + 1)];
      if (k == 0) sacc = mfma32_v_first(kf, qf[k]);
      else if (k == 35) mfma32_v_last(sacc, kf, qf[k]);
      else mfma32_v(sacc, kf, qf[k], ring[(k + AH) % (AH + 1)]);
      if (k + AH < 36) ring[(k + AH) % (AH + 1)] = qk_ld(k + AH);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Block 0 goes out now; the rest of the query (its 28 loads are the only
  // ones ahead of block 0's 9) is read while block 0 arrives.  Block 1 goes
  // out once block 0 is in and every wave is done with the query region:
  // drained together, the two would hold back the first scores by a whole
  // block's transfer.
  issue(0);
  asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  read_query(0, 28);
#pragma unroll
  for (int st = 0; st < 28; ++st) asm volatile("" : "+v"(qf[st]));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  issue(1);

  f32x16 x_unused;
  bf16x8 pb_unused[2], pb[2];
  // Top of iteration j: block j complete (block j + 1's 9 loads are the only
  // ones behind it) and every wave done with iteration j - 1.
  auto block_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    __syncthreads();
  };
  {
    // Block 0: its scores (block 2's gather going out beside them), then its
    // softmax on its own.
    const Gather g2 = gather_setup(2);
    f32x16 sacc;
    chain(0, sacc, &g2);
    const uint32_t vm = valid_mask(0);
    if (a.flags & 2u) write_scores(0, sacc, vm);
    const float cx = prepare(sacc, vm);
#pragma unroll
    for (int k = 0; k < kSoftSteps; ++k) soft_step(k, sacc, cx, pb);
  }
  // Iteration j: the score chain of block j, then the mix of block j - 1
  // with the softmax of block j and the gather of block j + 2 riding beside
  // its MFMAs.  pb holds block j - 1's P on entry, block j's on exit.
  for (int j = 1; j < nblk; ++j) {
    // Per-lane LDS bases are re-derived each iteration rather than kept as
    // dozens of hoisted base + offset sums occupying registers.
    asm volatile("" : "+v"(qk_base[0]), "+v"(qk_base[1]), "+v"(qk_base[2]), "+v"(qk_base[3]));
    asm volatile("" : "+v"(pc_base[0][0]), "+v"(pc_base[0][1]), "+v"(pc_base[1][0]), "+v"(pc_base[1][1]));
    block_barrier();
    const Gather gn = gather_setup(j + 2);
    const uint32_t vm = valid_mask(j);
    f32x16 sacc;
    chain(j, sacc, nullptr);
    // The factor decided by block j - 1's softmax, before its P is mixed in.
    if (resc_any) rescale(alpha);
    if (a.flags & 2u) write_scores(j, sacc, vm);
    const float cx = prepare(sacc, vm);
    bf16x8 pn[2];
    mix(std::true_type{}, j - 1, pb, sacc, cx, pn, &gn);
    pb[0] = pn[0];
    pb[1] = pn[1];
  }
  if (resc_any) rescale(alpha);
  mix(std::false_type{}, nblk - 1, pb, x_unused, 1.f, pb_unused, nullptr);

  // This lane's head: lanes l and l ^ 32 hold halves of the sum.
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  // The masked gathers past the last block may still be landing; after
  // this barrier the row buffers are free for the output tile.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // The wave's 32 heads go through LDS (tile row h = head h's 512 columns at
  // h * kTilePitch, the two 8-byte halves of each 16-byte chunk swapped when
  // bit 4 of h is set; with the padded pitch, the 32 heads of one store hit
  // distinct banks) so that the global writes are whole 1 KB rows.  With one split it is the normalised O~; with several,
  // each split stores its unnormalised sum with (max, sum) and the merge
  // applies 2^(m_s - M) / L.  One column tile at a time: the scheduling
  // barriers keep the accumulators from being read all at once.
  {
    const uint32_t half = 8u * (uint32_t)(hh ^ ((head >> 4) & 1));
    char* trow = smem + head * kTilePitch + half;
    const float inv = SPLIT ? 1.f : 1.0f / l_run;  // an empty selection gives 0 * inf = NaN
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = SPLIT ? acc[mt][4 * q4 + e] : acc[mt][4 * q4 + e] * inv;
        *reinterpret_cast<uint2*>(trow + 16 * (4 * mt + q4)) = pack4(o[0], o[1], o[2], o[3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (hh == 0 && head < a.H) {
      if constexpr (!SPLIT) {
        if (a.lse != nullptr)
          a.lse[(int64_t)b * a.H + head] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
        if (validate && !(l_run > 0.f)) atomicOr(a.status, 4u);
      } else {
        float* pml = a.part_ml + (((int64_t)s * a.B + b) * a.H + head) * 2;
        pml[0] = m_run;
        pml[1] = l_run;
      }
    }
  }
  // Row r of the wave's tile: lane l moves chunk l (the tile is the wave's
  // own, so no barrier: LDS operations of one wave complete in order).
#pragma unroll 8
  for (int r = 0; r < 32; ++r) {
    const int h = 32 * wave + r;
    if (h >= a.H) break;  // heads past a head-sharded call's share: not stored
    uint4 v = *reinterpret_cast<const uint4*>(smem + h * kTilePitch + 16 * lane);
    if (r & 16) v = uint4{v.z, v.w, v.x, v.y};
    *reinterpret_cast<uint4*>(dst + (int64_t)h * kLatent + 8 * lane) = v;
  }
}

// ---------------------------------------------------------------------------
// combine: O~ = sum_s g_s U_s, g_s = 2^(m_s - M) / L, L = sum_s 2^(m_s - M) l_s,
// where U_s is split s's unnormalised sum (relative to its max m_s).
// Workgroup = (sequence, 2 heads); each thread owns 4 latent columns.
// G = splits per group (2, 4 or 8, the smallest >= S up to 8).
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  const int hp = a.H / 2;  // head pairs per sequence
  const int b = (int)blockIdx.x / hp;
  const int head = ((int)blockIdx.x % hp) * 2 + (threadIdx.x >> 7);
  const int col = (threadIdx.x & 127) * 4;
  const int64_t stride_s = (int64_t)a.B * a.H;
  const int64_t bh = (int64_t)b * a.H + head;
  // Splits in groups of G whose loads are all in flight together (one at a
  // time, a 32-split merge is 32 memory latencies long); a group's slots past
  // S re-read split S - 1 (in bounds) and get weight 0.  The sums run over
  // s = 0 .. S - 1 in order.
  float M = -INFINITY;
  for (int s0 = 0; s0 < a.S; s0 += G) {
    float mv[G];
#pragma unroll
    for (int u = 0; u < G; ++u) mv[u] = a.part_ml[(min(s0 + u, a.S - 1) * stride_s + bh) * 2];
#pragma unroll
    for (int u = 0; u < G; ++u) M = fmaxf(M, mv[u]);
  }
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < a.S; s0 += G) {
    float2 ml[G];
    uint2 v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int64_t row = min(s0 + u, a.S - 1) * stride_s + bh;
      ml[u] = *reinterpret_cast<const float2*>(a.part_ml + row * 2);
      v[u] = *reinterpret_cast<const uint2*>(a.part_o + row * kLatent + col);
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      // Weight 0 for the unused slots (a select, not a branch, so that the
      // loads above stay ahead of all the arithmetic): their finite terms add
      // nothing.
      const bool used = s0 + u < a.S && ml[u].x != -INFINITY;
      const float w = used ? __builtin_amdgcn_exp2f(ml[u].x - M) : 0.f;
      L += w * ml[u].y;
      acc[0] += w * __uint_as_float(v[u].x << 16);
      acc[1] += w * __uint_as_float(v[u].x & 0xffff0000u);
      acc[2] += w * __uint_as_float(v[u].y << 16);
      acc[3] += w * __uint_as_float(v[u].y & 0xffff0000u);
    }
  }
  const float inv = 1.0f / L;
  *reinterpret_cast<uint2*>(a.o_latent + bh * kLatent + col) =
      pack4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if ((threadIdx.x & 127) == 0) {
    if (a.lse != nullptr) a.lse[bh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    if (a.status != nullptr && head == 0 && !(L > 0.f)) atomicOr(a.status, 4u);
  }
}

// ---------------------------------------------------------------------------
// output projection ("Attention update" page, mla-output): each sequence's
// head outputs flattened (i = 128 h + d) and projected to the model width,
//   out[b][o] = sum_i x[b][i] wo[o][i],  wo [7168][16384] (a linear weight).
// HBM-bound on wo (235 MB, read once per launch of up to 64 batch rows).
// Workgroup = 28 output features (7168 = 256 x 28: one workgroup per CU),
// padded to the 32 rows of an MFMA tile (rows past 28 lie outside the weight
// range and load zeros).  K = i is walked in chunks of 256; wave w takes
// line w of every chunk (its 64 columns: K-steps 4w .. 4w + 3), so each
// wave moves, by whole-line LDS-DMA into three buffers of its own, exactly
// the 128-byte lines it reads: the 32 wo rows' and the x rows' line w of
// the chunk, two chunks ahead.  The waves never wait for each other until
// the end, where their sums are added through LDS.  Line of row r at
// segment r (wo) or 32 + r (x) of a buffer, 16-byte chunk q at position
// q ^ seg_swz(r): the fragment reads of 32 rows at one chunk hit distinct
// banks.  M = o (A fragments), N = b (B fragments), K = i.  Each CU ingests
// all of x (2 MB at B = 64, twice its 0.9 MB of wo), which with two chunks
// in flight per wave is what sets the rate at large batches.
// ---------------------------------------------------------------------------
constexpr int kOpRows = 28;        // output features per workgroup
constexpr int kOpChunk = 256;      // K per chunk: four 64-column lines

// PACKED: wo in the layout of mla_output_proj_pack, where workgroup g's 28
// rows are stored chunk by chunk ([chunk][row][256 columns]), so that each
// chunk's weight lines are one contiguous 14 KB piece; the same bytes reach
// the same LDS slots either way.
template <int NT, bool PACKED>
__global__ __launch_bounds__(256, 1) void output_proj_kernel(const OutProjArgs a) {
  constexpr int XR = 32 * NT;                    // x rows staged per chunk
  constexpr int kSegs = 32 + XR;                 // 128-byte segments per buffer
  constexpr int kWaveLds = 3 * kSegs * 128;      // three buffers per wave
  constexpr int kDpc = 4 + XR / 8;               // DMA instructions per wave per chunk
  constexpr int kChunks = kWoIn / kOpChunk;      // 64
  static_assert((kChunks & (kChunks - 1)) == 0, "the chunk walk wraps with a mask");
  __shared__ __attribute__((aligned(1024))) char smem[4 * kWaveLds];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int o0 = kOpRows * (int)blockIdx.x;
  char LDS_AS* wl = (char LDS_AS*)smem + wave * kWaveLds;
  const uint32_t lds_w = (uint32_t)(uintptr_t)wl;
  const i32x4 rw = buffer_rsrc(a.wo + (size_t)o0 * kWoIn, (uint32_t)(kOpRows * kWoIn * 2));
  const i32x4 rx = buffer_rsrc(a.x, (uint32_t)(((int64_t)(a.B - 1) * a.x_sb + kWoIn) * 2));
  const uint32_t r8 = (uint32_t)(lane >> 3);
  // Workgroup x walks K from chunk x / 8 on (wrapping round): were every
  // workgroup at the same chunk, the plain layout's weight reads (pieces of
  // rows 32 KB apart, all at one column offset) would crowd into the same
  // memory channels; staggered, it reads as fast as the packed layout.  The
  // packed layout takes the same order, so the two give identical sums.
  const int c_first = (int)blockIdx.x >> 3;
  // Step it's chunk c = (c_first + it) mod 64 into buffer it % 3: instruction j
  // moves rows 8j .. 8j + 7 (lane l: row 8j + l / 8, position l % 8, source
  // chunk (l % 8) ^ seg_swz(row)).
  auto issue = [&](int it) __attribute__((always_inline)) {
    const uint32_t buf = lds_w + (uint32_t)((it % 3) * kSegs * 128);
    const int c = (c_first + it) & (kChunks - 1);
    const uint32_t col = (uint32_t)(c * kOpChunk + 64 * wave) * 2u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t r = (uint32_t)(8 * j) + r8;
      const uint32_t q16 = (((uint32_t)(lane & 7)) ^ seg_swz(r)) * 16u;
      const uint32_t off = PACKED ? (r < (uint32_t)kOpRows
                                         ? ((uint32_t)c * kOpRows + r) * (uint32_t)(kOpChunk * 2) +
                                               (uint32_t)(128 * wave) + q16
                                         : kMaskedOffset)
                                  : r * (uint32_t)(kWoIn * 2) + col + q16;
      dma16(rw, buf + (uint32_t)(8 * j) * 128u, off);
    }
#pragma unroll
    for (int j = 0; j < XR / 8; ++j) {
      const uint32_t r = (uint32_t)(8 * j) + r8;
      const uint32_t q16 = (((uint32_t)(lane & 7)) ^ seg_swz(r)) * 16u;
      dma16(rx, buf + (uint32_t)(32 + 8 * j) * 128u, r * (uint32_t)(a.x_sb * 2) + col + q16);
    }
  };
  // Fragment of K-step t (0..3) of the wave's line: row `row` of segment
  // base `seg0`, chunk 2 t + hh.
  const uint32_t r32 = (uint32_t)(lane & 31);
  auto frag = [&](const char LDS_AS* buf, uint32_t seg0, int t) __attribute__((always_inline)) {
    const uint32_t q = (uint32_t)(2 * t + hh);
    return *(const bf16x8 LDS_AS*)(buf + (seg0 + r32) * 128u + ((q ^ seg_swz(r32)) * 16u));
  };

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  issue(0);
  issue(1);
  for (int it = 0; it < kChunks; ++it) {
    // Step it's chunk has landed when at most step it + 1's loads are outstanding.
    if (it + 1 < kChunks) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDpc) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // Buffer (it + 2) % 3 last held step it - 1's chunk, whose fragments were
    // read (and used) in the previous iteration.
    if (it + 2 < kChunks) issue(it + 2);
    const char LDS_AS* buf = wl + (it % 3) * kSegs * 128;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 af = frag(buf, 0u, t);
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = mfma32(af, frag(buf, (uint32_t)(32 + 32 * n), t), acc[n]);
    }
  }

  // acc[n][v] of lane l: output feature o0 + 8 (v / 4) + 4 (l / 32) + v % 4,
  // batch row 32 n + l % 32.  Each wave's sums into its own LDS region, then
  // every thread adds the four waves' values of 8 outputs.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float* red = reinterpret_cast<float*>(smem + wave * kWaveLds);
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[(n * 16 + v) * 64 + lane] = acc[n][v];
  __syncthreads();
  for (int e = tid; e < NT * 16 * 64; e += 256) {
    const int n = e >> 10, v = (e >> 6) & 15, l = e & 63;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) sum += reinterpret_cast<const float*>(smem + w * kWaveLds)[e];
    const int m = 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    const int b = 32 * n + (l & 31);
    if (m < kOpRows && b < a.B)
      a.out[(int64_t)b * a.out_sb + o0 + m] = __builtin_bit_cast(uint16_t, (__bf16)sum);
  }
}

// ---------------------------------------------------------------------------
// Output projection split over the inputs (mla_output_proj_split): each CU
// of output_proj_kernel ingests all of x (2 MB at B = 64, twice its 0.9 MB of
// wo), and at large batches that sets the rate.  Here workgroup (g, q) takes
// 112 outputs (four 28-row tiles, tile w for wave w) over input quarter q
// (4096 inputs), so a CU ingests a quarter of x beside the same 0.9 MB of wo;
// the four quarters' fp32 partial sums go to a workspace and
// output_proj_reduce_kernel adds them in quarter order.  K is walked in
// chunks of 128 (two 128-byte lines per row): per chunk, wave w moves its
// tile's 32 weight rows (rows past 28 masked) and a quarter of the x lines by
// whole-line LDS-DMA into one of three buffers, two chunks ahead; the x lines
// are shared by the four waves, so each chunk ends with a barrier.  Units are
// numbered XCD-major: an XCD runs eight groups' four quarters, so each x
// quarter is read by eight of its workgroups through its L2; and the
// workgroups of XCD x start their walk at chunk 4 x (wrapping round), so that
// the eight XCDs read different columns of wo at any moment while the
// workgroups of one XCD read the same x lines together.  Line l of row r at
// segment l * R + r of its region (R = 32 rows per wo tile, 32 NT x rows),
// 16-byte chunk c at position c ^ seg_swz(r).  M = o, N = b, K = i.
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256, 1) void output_proj_split_kernel(const OutProjArgs a) {
  constexpr int XR = 32 * NT;                    // x rows staged per chunk
  constexpr int kQK = kWoIn / kOpSplit;          // 4096 inputs per quarter
  constexpr int kNch = kQK / 128;                // 32 chunks
  constexpr int kWoSegs = 4 * 64;                // four tiles x 2 lines x 32 rows
  constexpr int kBufSegs = kWoSegs + 2 * XR;     // + 2 lines x XR rows of x
  constexpr int kDpc = 8 + XR / 16;              // DMA instructions per wave per chunk
  static_assert((kNch & (kNch - 1)) == 0, "the chunk walk wraps with a mask");
  __shared__ __attribute__((aligned(1024))) char smem[3 * kBufSegs * 128];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int x8 = (int)blockIdx.x;
  const int u = (x8 & 7) * 32 + (x8 >> 3);       // XCD-major unit
  const int g = u >> 2, q = u & 3;               // output group, input quarter
  const int o0 = 4 * kOpRows * g + kOpRows * wave;  // this wave's tile
  const uint32_t lds0 = (uint32_t)(uintptr_t)(char LDS_AS*)smem;
  const i32x4 rw = buffer_rsrc(a.wo + (size_t)o0 * kWoIn + (size_t)q * kQK,
                               (uint32_t)(((kOpRows - 1) * kWoIn + kQK) * 2));
  const i32x4 rx = buffer_rsrc(a.x + (size_t)q * kQK, (uint32_t)(((int64_t)(a.B - 1) * a.x_sb + kQK) * 2));
  const int c_first = (x8 & 7) * 4;
  // Step it's chunk c into buffer it % 3.  Weight: instruction j moves lines
  // 8j .. 8j + 7 of the tile (line li: row li % 32, half li / 32; lane l takes
  // line 8j + l / 8, position l % 8).  x: wave w moves lines XR/2 w .. of the
  // 2 XR (line li: row li % XR, half li / XR).
  auto issue = [&](int it) __attribute__((always_inline)) {
    const int c = (c_first + it) & (kNch - 1);
    const uint32_t buf = lds0 + (uint32_t)((it % 3) * kBufSegs * 128);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t li = (uint32_t)(8 * j) + (uint32_t)(lane >> 3);
      const uint32_t r = li & 31u, l = li >> 5;
      const uint32_t q16 = (((uint32_t)(lane & 7)) ^ seg_swz(r)) * 16u;
      dma16(rw, buf + (uint32_t)(wave * 64 + 8 * j) * 128u,
            r * (uint32_t)(kWoIn * 2) + (uint32_t)(c * 256) + l * 128u + q16);
    }
#pragma unroll
    for (int j = 0; j < XR / 16; ++j) {
      const uint32_t li = (uint32_t)(wave * (XR / 2) + 8 * j) + (uint32_t)(lane >> 3);
      const uint32_t b = li & (uint32_t)(XR - 1), l = li / (uint32_t)XR;
      const uint32_t q16 = (((uint32_t)(lane & 7)) ^ seg_swz(b)) * 16u;
      dma16(rx, buf + (uint32_t)(kWoSegs + wave * (XR / 2) + 8 * j) * 128u,
            b * (uint32_t)(a.x_sb * 2) + (uint32_t)(c * 256) + l * 128u + q16);
    }
  };
  // Fragment of K-step st (0..7) of a chunk: row `row` at segment `seg`,
  // 16-byte chunk 2 (st % 4) + hh of its line.
  const uint32_t r32 = (uint32_t)(lane & 31);
  auto frag = [&](const char LDS_AS* buf, uint32_t seg, uint32_t row, int st) __attribute__((always_inline)) {
    const uint32_t c = (uint32_t)(2 * (st & 3) + hh);
    return *(const bf16x8 LDS_AS*)(buf + seg * 128u + ((c ^ seg_swz(row)) * 16u));
  };

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  issue(0);
  issue(1);
  for (int it = 0; it < kNch; ++it) {
    // This wave's loads of step it are in when at most step it + 1's are
    // outstanding; after the barrier every wave's are, and every wave is done
    // with buffer (it + 2) % 3, read in the previous step.
    if (it + 1 < kNch) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDpc) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 2 < kNch) issue(it + 2);
    const char LDS_AS* buf = (const char LDS_AS*)smem + (it % 3) * kBufSegs * 128;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const uint32_t l = (uint32_t)(st >> 2);
      const bf16x8 af = frag(buf, (uint32_t)(wave * 64) + l * 32u + r32, r32, st);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint32_t b = (uint32_t)(32 * n) + r32;
        acc[n] = mfma32(af, frag(buf, (uint32_t)kWoSegs + l * (uint32_t)XR + b, b, st), acc[n]);
      }
    }
  }
  // acc[n][v] of lane l: output o0 + 8 (v / 4) + 4 (l / 32) + v % 4, batch row
  // 32 n + l % 32; four consecutive outputs per store.
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int b = 32 * n + (lane & 31);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int m = 8 * g4 + 4 * hh;
      if (m < kOpRows && b < a.B)
        *reinterpret_cast<float4*>(a.part + ((int64_t)q * a.B + b) * kWoOut + o0 + m) =
            float4{acc[n][4 * g4], acc[n][4 * g4 + 1], acc[n][4 * g4 + 2], acc[n][4 * g4 + 3]};
    }
  }
}

// The quarters' partial sums of 4 consecutive outputs per thread (one
// 16-byte load per quarter, all four in flight together), added in quarter
// order and rounded to bf16.
__global__ __launch_bounds__(256) void output_proj_reduce_kernel(const OutProjArgs a) {
  constexpr int kPer = kWoOut / 4;
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (i >= a.B * kPer) return;
  const int b = i / kPer, o = (i % kPer) * 4;
  float4 v[kOpSplit];
#pragma unroll
  for (int qq = 0; qq < kOpSplit; ++qq)
    v[qq] = *reinterpret_cast<const float4*>(a.part + ((int64_t)qq * a.B + b) * kWoOut + o);
  float4 s = v[0];
#pragma unroll
  for (int qq = 1; qq < kOpSplit; ++qq) {
    s.x += v[qq].x;
    s.y += v[qq].y;
    s.z += v[qq].z;
    s.w += v[qq].w;
  }
  uint16_t* dst = a.out + (int64_t)b * a.out_sb + o;
  dst[0] = __builtin_bit_cast(uint16_t, (__bf16)s.x);
  dst[1] = __builtin_bit_cast(uint16_t, (__bf16)s.y);
  dst[2] = __builtin_bit_cast(uint16_t, (__bf16)s.z);
  dst[3] = __builtin_bit_cast(uint16_t, (__bf16)s.w);
}

// ---------------------------------------------------------------------------
// Output-projection weight repack (one-time set-up): packed[g][c][r][k] =
// wo[28 g + r][256 c + k] for the 256 workgroups g, 64 chunks c, 28 rows r
// and 256 columns k, 16 bytes per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void output_proj_pack_kernel(const uint16_t* __restrict__ wo,
                                                               uint16_t* __restrict__ packed) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;  // packed element index
  const int k = (int)(i % kOpChunk);
  const size_t rest = i / kOpChunk;
  const int r = (int)(rest % kOpRows);
  const size_t gc = rest / kOpRows;
  const int c = (int)(gc % (kWoIn / kOpChunk));
  const int g = (int)(gc / (kWoIn / kOpChunk));
  const size_t src = (size_t)(kOpRows * g + r) * kWoIn + (size_t)c * kOpChunk + k;
  *reinterpret_cast<uint4*>(packed + i) = *reinterpret_cast<const uint4*>(wo + src);
}

// ---------------------------------------------------------------------------
// fp8 dequantisation (one-time set-up): the whole weight, with the helpers
// above.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_kernel(const DequantArgs a) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  const int row = (int)(i / kLatent), col = (int)(i % kLatent);
  const float sc = a.scales[(row / 128) * (kLatent / 128) + col / 128];
  const uint2 codes = *reinterpret_cast<const uint2*>(a.w + i);
  uint32_t outw[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    uint32_t pair = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t word = (e + k) < 4 ? codes.x : codes.y;
      const uint32_t code = (word >> (8 * ((e + k) & 3))) & 0xffu;
      const float v = e4m3_value(code);
      const float p = v * sc;
      const float err = __builtin_fmaf(v, sc, -p);
      pair |= bf16_rne_exact(p, err) << (16 * k);
    }
    outw[e / 2] = pair;
  }
  *reinterpret_cast<uint4*>(a.out + i) = uint4{outw[0], outw[1], outw[2], outw[3]};
}

}  // namespace

int launch_absorb(const AbsorbArgs& a, void* stream) {
  if (a.fp8.w_fp8 != nullptr)
    hipLaunchKernelGGL(absorb_kernel<true>, dim3(a.H * 2), dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(absorb_kernel<false>, dim3(a.H * 2), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_decode(const DecodeArgs& a, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  // Whole XCD rounds; spare workgroups exit.  Prefill deals whole rows (all
  // their splits) to each XCD in turn.
  const int grid = a.causal ? 8 * ((a.B + 7) / 8) * a.S : 8 * ((a.B * a.S + 7) / 8);
  auto* k = a.indices == nullptr ? (a.S > 1 ? decode_kernel<true, true> : decode_kernel<true, false>)
                                  : (a.S > 1 ? decode_kernel<false, true> : decode_kernel<false, false>);
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

int launch_output_proj(const OutProjArgs& a, void* stream) {
  static_assert(kWoOut % kOpRows == 0, "whole output tiles");
  const dim3 grid(kWoOut / kOpRows);
  const hipStream_t st = (hipStream_t)stream;
  if (a.packed) {
    if (a.B <= 32) hipLaunchKernelGGL((output_proj_kernel<1, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((output_proj_kernel<2, true>), grid, dim3(256), 0, st, a);
  } else {
    if (a.B <= 32) hipLaunchKernelGGL((output_proj_kernel<1, false>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((output_proj_kernel<2, false>), grid, dim3(256), 0, st, a);
  }
  return (int)hipGetLastError();
}

int launch_output_proj_split(const OutProjArgs& a, void* stream) {
  static_assert(kWoOut == 64 * 4 * kOpRows, "64 groups of four output tiles");
  const hipStream_t st = (hipStream_t)stream;
  if (a.B <= 32) hipLaunchKernelGGL((output_proj_split_kernel<1>), dim3(256), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((output_proj_split_kernel<2>), dim3(256), dim3(256), 0, st, a);
  hipLaunchKernelGGL(output_proj_reduce_kernel, dim3((unsigned)((a.B * (kWoOut / 4) + 255) / 256)), dim3(256), 0, st,
                     a);
  return (int)hipGetLastError();
}

int launch_output_proj_pack(const uint16_t* wo, uint16_t* packed, void* stream) {
  constexpr size_t n = (size_t)kWoOut * kWoIn;
  static_assert(n % (256 * 8) == 0, "whole workgroups");
  hipLaunchKernelGGL(output_proj_pack_kernel, dim3((unsigned)(n / (256 * 8))), dim3(256), 0, (hipStream_t)stream,
                     wo, packed);
  return (int)hipGetLastError();
}

int launch_combine(const CombineArgs& a, void* stream) {
  const dim3 grid(a.B * (a.H / 2));
  if (a.S <= 2) hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(256), 0, (hipStream_t)stream, a);
  else if (a.S <= 4) hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(256), 0, (hipStream_t)stream, a);
  else hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

template <bool FP8>
static void launch_value_up_t(const ValueUpArgs& a, dim3 grid, bool small, bool two, hipStream_t st) {
  if (a.o_latent == nullptr) {
    if (small) {
      if (two) hipLaunchKernelGGL((value_up_kernel<true, 16, 2, FP8>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((value_up_kernel<true, 16, 4, FP8>), grid, dim3(256), 0, st, a);
    } else {
      if (two) hipLaunchKernelGGL((value_up_kernel<true, 32, 2, FP8>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((value_up_kernel<true, 32, 4, FP8>), grid, dim3(256), 0, st, a);
    }
  } else {
    if (small) hipLaunchKernelGGL((value_up_kernel<false, 16, 2, FP8>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((value_up_kernel<false, 32, 2, FP8>), grid, dim3(256), 0, st, a);
  }
}

int launch_value_up(const ValueUpArgs& a, void* stream) {
  if (a.o_latent != nullptr && a.B >= kValueUpStreamMinRows) {
    // Merged rows at large batches: W_UV,h formed once per workgroup, the
    // tiles streamed; enough workgroups per head to give every CU one.
    const int ntiles = (a.B + 31) / 32;
    const int groups = max(1, min(ntiles, (256 + a.H - 1) / a.H));
    const int units = a.H * groups;
    const dim3 grid(8 * ((units + 7) / 8));
    const hipStream_t st = (hipStream_t)stream;
    if (a.fp8.w_fp8 != nullptr) hipLaunchKernelGGL(value_up_stream_kernel<true>, grid, dim3(256), 0, st, a, groups);
    else hipLaunchKernelGGL(value_up_stream_kernel<false>, grid, dim3(256), 0, st, a, groups);
    return (int)hipGetLastError();
  }
  // 32-row tiles, or 16 when that is what it takes to give every CU a tile.
  // Two splits staged per pass when there are at most two (half the LDS, so
  // two workgroups fit a CU), else four.
  const bool small = a.B <= 32;
  const int rows = small ? 16 : 32;
  const bool two = a.o_latent != nullptr || a.S <= 2;
  const int units = a.H * ((a.B + rows - 1) / rows);
  const dim3 grid(8 * ((units + 7) / 8));
  const hipStream_t st = (hipStream_t)stream;
  if (a.fp8.w_fp8 != nullptr) launch_value_up_t<true>(a, grid, small, two, st);
  else launch_value_up_t<false>(a, grid, small, two, st);
  return (int)hipGetLastError();
}

int launch_dequant(const DequantArgs& a, void* stream) {
  const size_t n = (size_t)kHeads * kRowsPerHead * kLatent;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)(n / 8 / 256)), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int device_cu_count(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  return (int)hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (mla_sparse_decode_noalloc):
// the split partials live in this file-scope device array, one copy per GPU,
// held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in symbol): the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept here.
// ---------------------------------------------------------------------------
namespace {
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
int g_scratch_err[kMaxDevices];
}  // namespace

int scratch_buffer(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = (int)r;
    g_scratch_ptr[dev] = r == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != 0) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return 0;
}

}  // namespace mla
