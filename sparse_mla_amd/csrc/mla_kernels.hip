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

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// Four floats -> four bf16 (round to nearest even), packed for an 8-byte store.
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  uint2 r;
  r.x = (uint32_t)bf16_bits(a) | ((uint32_t)bf16_bits(b) << 16);
  r.y = (uint32_t)bf16_bits(c) | ((uint32_t)bf16_bits(d) << 16);
  return r;
}

// ---------------------------------------------------------------------------
// absorb: q_abs[b][h][c] = sum_d q_nope[b][h][d] W_UK,h[d][c]
// Workgroup = (head, 256-column half): 256 workgroups, each streaming its
// 64 KB slab of W_UK once and looping over 32-row batch tiles.  W_UK is
// stored [d][c] (c contiguous)
// while d is the reduction index, so the 128 x 256 slab (64 KB) is moved into
// LDS by LDS-DMA -- 8 lanes per 128-byte line, line m of row d at segment
// (m * 128 + d), chunk q at 16-byte position q ^ 2 (d % 4), which keeps the
// transpose reads conflict-free -- and read back as K-strided MFMA fragments.
// Wave w owns columns 64 w .. 64 w + 63 of the half (two 32-column tiles):
// M = c, N = b, K = d.  The first query tiles load while the slab is in flight.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void absorb_kernel(const AbsorbArgs a) {
  __shared__ __attribute__((aligned(1024))) char wt[4 * kNope * 128];
  const int h = blockIdx.x & (kHeads - 1);
  const int ch = blockIdx.x >> 7;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, i16 = lane & 15, gm = (lane >> 4) & 1;
  const char LDS_AS* wl = (const char LDS_AS*)wt;
  {
    const i32x4 rw = buffer_rsrc(a.wkv_b + (size_t)h * kRowsPerHead * kLatent + ch * 256,
                                 (uint32_t)((kNope - 1) * kLatent * 2 + 512));
    const uint32_t lds0 = (uint32_t)(uintptr_t)wl;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int ins = wave * 16 + k;                   // line ins / 16, rows 8 (ins % 16) + 0..7
      const uint32_t d = (uint32_t)(((ins & 15) << 3) + (lane >> 3));
      const uint32_t q = (uint32_t)(lane & 7) ^ (2u * (d & 3u));
      dma16(rw, lds0 + (uint32_t)ins * 1024u, d * (uint32_t)(kLatent * 2) + (uint32_t)(ins >> 4) * 128u + q * 16u);
    }
  }
  // A operand (the slab, as K-strided fragments) is the same for every batch
  // tile: read it once.  Query tiles are loaded four at a time.
  const int nbt = (a.B + 31) / 32;
  bf16x8 qb[4][8];
  auto load_q = [&](int bt0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // Rows past B load row B-1: they only feed output columns that are
      // never stored, and unconditional loads keep all of them in flight.
      const int bb = min((bt0 + u) * 32 + (lane & 31), a.B - 1);
      const uint16_t* q = a.q_nope + (int64_t)bb * a.q_sb + (int64_t)h * a.q_sh + 8 * hh;
#pragma unroll
      for (int st = 0; st < 8; ++st) qb[u][st] = ld8(q + 16 * st);
    }
  };
  load_q(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  bf16x8 af[2][8];
#pragma unroll
  for (int st = 0; st < 8; ++st)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t off[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint32_t d = (uint32_t)(16 * st + 8 * hh + 4 * r + (i16 >> 2));
        const uint32_t q = (uint32_t)(4 * t + 2 * gm + ((i16 & 3) >> 1));
        off[r] = ((uint32_t)wave * kNope + d) * 128u + ((q ^ (2u * (d & 3u))) * 16u) + 8u * (uint32_t)(i16 & 1);
      }
      af[t][st] = tr_pair(wl + off[0], wl + off[1]);
    }
  for (int bt0 = 0; bt0 < nbt; bt0 += 4) {
    if (bt0 > 0) load_q(bt0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int bb = (bt0 + u) * 32 + (lane & 31);
      if (bt0 + u >= nbt) break;
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = mfma32(af[t][st], qb[u][st], acc[t]);
      if (bb < a.B) {
        uint16_t* o = a.q_abs + ((int64_t)bb * kHeads + h) * kLatent + ch * 256 + wave * 64 + 4 * hh;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<uint2*>(o + 32 * t + 8 * q4) =
                pack4(acc[t][4 * q4], acc[t][4 * q4 + 1], acc[t][4 * q4 + 2], acc[t][4 * q4 + 3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// value-up: out[b][h][d] = sum_c O~[b][h][c] W_UV,h[d][c]
// Workgroup = head: 128 workgroups, each reading its 128 KB of W_UV once
// (wave w keeps value rows 32 w .. 32 w + 31 in registers) and looping over
// 32-row batch tiles.  Each O~ tile [32][512] is assembled in LDS (rows
// padded to 1040 bytes, two buffers alternating), then wave w computes
// value rows 32 w .. 32 w + 31: M = d (W_UV rows, contiguous along c, loaded
// straight into registers while the tile is assembled), N = b (from LDS),
// K = c.  FUSED: the tile is merged from the split partials of the decode
// ("Softmax" page, normalisation over all selected keys):
//   O~ = sum_s g_s O~_s, g_s = 2^(m_s - M) l_s / L, L = sum_s 2^(m_s - M) l_s,
//   lse = ln 2 (M + log2 L)
// ---------------------------------------------------------------------------
constexpr int kOtRow = 1040;  // bytes per O~ row in LDS (512 bf16 + 16 pad)

template <bool FUSED>
__global__ __launch_bounds__(256) void value_up_kernel(const ValueUpArgs a) {
  __shared__ __attribute__((aligned(16))) char ot[2][32 * kOtRow];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t* w = a.wkv_b + ((size_t)h * kRowsPerHead + kNope + 32 * wave + (lane & 31)) * kLatent + 8 * hh;
  bf16x8 wf[32];
#pragma unroll
  for (int st = 0; st < 32; ++st) wf[st] = ld8(w + 16 * st);

  const int nbt = (a.B + 31) / 32;
  for (int bt = 0; bt < nbt; ++bt) {
  char* tile = ot[bt & 1];
  // O~ tile: wave w fills rows 8 w .. 8 w + 7; lane l owns columns
  // 8 l .. 8 l + 7 of each row (one coalesced 1 KB line per load).  All loads
  // of a pass are issued before any of them is used; rows past B read row
  // B-1 and are written as zeros.
  int64_t bh[8];
  bool okr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int bb = bt * 32 + 8 * wave + j;
    okr[j] = bb < a.B;
    bh[j] = (int64_t)min(bb, a.B - 1) * kHeads + h;
  }
  float v[8][8];
  if constexpr (FUSED) {
    // Lane s holds split s's (max, sum); the merge weights come from two wave
    // reductions per row and are broadcast to all lanes.
    const int64_t sstride = (int64_t)a.B * kHeads;
    const int ls = min(lane, a.S - 1);
    float2 ml[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ml[j] = *reinterpret_cast<const float2*>(a.part_ml + ((int64_t)ls * sstride + bh[j]) * 2);
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float m = lane < a.S ? ml[j].x : -INFINITY;
      float M = m;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
      const float e = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M) * ml[j].y;
      float L = e;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
      g[j] = e / L;
      const float empty = L > 0.f ? 0.f : __builtin_nanf("");  // all -inf row: NaN, as in mla_combine
#pragma unroll
      for (int k = 0; k < 8; ++k) v[j][k] = empty;
      if (lane == 0 && okr[j]) {
        if (a.lse != nullptr) a.lse[bh[j]] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
        if (a.status != nullptr && h == 0 && !(L > 0.f)) atomicOr(a.status, 4u);
      }
    }
    for (int s0 = 0; s0 < a.S; s0 += 2) {
      bf16x8 x[8][2];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          x[j][u] = ld8(a.part_o + ((int64_t)min(s0 + u, a.S - 1) * sstride + bh[j]) * kLatent + 8 * lane);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float gs = (s0 + u < a.S) ? __shfl(g[j], s0 + u) : 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) v[j][k] += gs * (float)x[j][u][k];
        }
    }
  } else {
    bf16x8 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = ld8(a.o_latent + bh[j] * kLatent + 8 * lane);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) v[j][k] = (float)x[j][k];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bf16x8 y;
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = okr[j] ? (__bf16)v[j][k] : (__bf16)0.f;
    *reinterpret_cast<bf16x8*>(tile + (8 * wave + j) * kOtRow + 16 * lane) = y;
  }
  __syncthreads();

  f32x16 acc = {};
  const char LDS_AS* ol = (const char LDS_AS*)tile + (lane & 31) * kOtRow + 16 * hh;
#pragma unroll
  for (int st = 0; st < 32; ++st) acc = mfma32(wf[st], *(const bf16x8 LDS_AS*)(ol + 32 * st), acc);
  const int bb = bt * 32 + (lane & 31);
  if (bb < a.B) {
    uint16_t* out = a.out + (int64_t)bb * a.out_sb + (int64_t)h * a.out_sh + 32 * wave + 4 * hh;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<uint2*>(out + 8 * q4) = pack4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
  }
  }  // batch tiles (two tile buffers: one barrier per tile suffices)
}

// ---------------------------------------------------------------------------
// decode: sparse flash-decode over the selected cache rows.
//
// Workgroup = (sequence b, head group, key split); 4 waves.  With KL key lanes
// (head_groups == KL), a workgroup covers 128 / KL heads as 4 / KL slices of
// 32 heads; wave w = (slice w / KL, key lane w % KL).  Each block of
// NKEY = 32 KL keys is gathered into LDS by buffer loads that write LDS
// directly (16 bytes per lane, one 1 KiB line per instruction), NBUF blocks
// in flight.  Masked slots get an offset past the record range, so their
// rows arrive as zeros.
//
// LDS block layout: a row [latent 512 | rotary 64] is 9 lines of 128 bytes
// (8 chunks of 8 features each).  Line m of key k is the 128-byte segment
// (m * NKEY + k) * 128, and chunk q of that line sits at 16-byte position
// q ^ sw(k).  One gather instruction moves 8 segments (8 keys, one line
// each): 8 adjacent lanes read one whole 128-byte line of one row.  sw() is
// chosen so that the score reads (32 keys, one chunk) and the transpose
// reads (8 keys x 4 chunks) hit distinct banks for 32- and 64-bank LDS.
//
// Per wave and block of 32 keys:
//   scores  S^T[key][head] = sum_f row[key][f] Q~[head][f]: A = rows (LDS,
//           ds_read_b128), B = [q~ | q_pe] (registers), M = keys, N = heads,
//           36 MFMAs over the 576 features.
//   softmax each lane holds 16 keys of one head: in-lane max/sum plus one
//           exchange with lane ^ 32; exp2 with the scale folded into log2 e.
//   mix     O~^T[col][head] += sum_key C[key][col] P[head][key]: A = latent
//           columns via transpose reads (M = 512 columns in 16 tiles), B = P
//           taken from the score registers in place (K = keys, permuted
//           consistently on both sides), N = heads.  Every accumulator of a
//           lane belongs to its own head, so rescaling needs no exchange.
// ---------------------------------------------------------------------------
template <int KL, int NBUF, bool DENSE>
__global__ __launch_bounds__(256, 1) void decode_kernel(const DecodeArgs a) {
  constexpr int NKEY = 32 * KL;
  constexpr int HPW = 128 / KL;                 // heads per workgroup
  constexpr int BUF = 72 * NKEY * 16;           // bytes per block buffer
  constexpr int GPW = BUF / 1024 / 4;           // gather instructions per wave per block
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * BUF + kIdxCap * 4];
  char LDS_AS* s3 = (char LDS_AS*)smem;
  int* sidx = reinterpret_cast<int*>(smem + NBUF * BUF);

  // Workgroup -> (sequence, split, head group).  Dispatch places workgroup i
  // on XCD i % 8; the head groups of one (sequence, split) are given ids 8
  // apart so they share an XCD (and its L2) and start together.
  const int wg = blockIdx.x;
  const int x8 = wg & 7, y = wg >> 3;
  const int hg = y % KL;
  const int unit = (y / KL) * 8 + x8;
  if (unit >= a.B * a.S) return;
  const int b = unit / a.S, s = unit % a.S;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = wave / KL, kl = wave % KL;
  const int hh = lane >> 5;
  const int head = hg * HPW + hs * 32 + (lane & 31);

  constexpr bool dense = DENSE;
  const bool validate = (a.flags & 1u) != 0 && hg == 0;
  const int Lb = min(max(a.seq_lens[b], 0), a.max_len);
  const int s0 = s * a.chunk;
  const int s1 = min(a.k_max, s0 + a.chunk);
  const int nslot = max(0, s1 - s0);
  const int nblk = (nslot + NKEY - 1) / NKEY;

  // Query operand [q~ (512) | q_pe (64)] for this lane's head, in MFMA B layout.
  bf16x8 qf[36];
  auto load_query = [&]() {
    const uint16_t* qa = a.q_abs + ((int64_t)b * kHeads + head) * kLatent + 8 * hh;
#pragma unroll
    for (int st = 0; st < 32; ++st) qf[st] = ld8(qa + 16 * st);
    const uint16_t* qp = a.q_pe + (int64_t)b * a.q_pe_sb + (int64_t)head * a.q_pe_sh + 8 * hh;
#pragma unroll
    for (int st = 0; st < 4; ++st) qf[32 + st] = ld8(qp + 16 * st);
  };

  // Stage this split's index slots as cache rows (-1 = masked).  The same
  // predicate decides validity, the attended bitmap and the device checks.
  // Thread t owns slots 4 t .. 4 t + 3 of each 1024-slot pass; all of its
  // loads are issued before any is used.
  if constexpr (!dense) {
    constexpr int kPass = 4 * 256;
    int4 raw[kIdxCap / kPass];
#pragma unroll
    for (int ps = 0; ps < kIdxCap / kPass; ++ps) {
      const int i0 = ps * kPass + 4 * tid;
      const int64_t base = (int64_t)b * a.k_max + s0 + i0;
      if (i0 + 3 < nslot && (base & 3) == 0) {
        raw[ps] = *reinterpret_cast<const int4*>(a.indices + base);
      } else {
        raw[ps].x = i0 + 0 < nslot ? a.indices[base + 0] : -1;
        raw[ps].y = i0 + 1 < nslot ? a.indices[base + 1] : -1;
        raw[ps].z = i0 + 2 < nslot ? a.indices[base + 2] : -1;
        raw[ps].w = i0 + 3 < nslot ? a.indices[base + 3] : -1;
      }
    }
    // The query operand loads go out after the index loads and stay in
    // flight: vmcnt retires in order, so waiting for the indices leaves the
    // 36 query loads outstanding, and the first block's wait covers them.
    load_query();
    asm volatile("s_waitcnt vmcnt(36)" ::: "memory");
#pragma unroll
    for (int ps = 0; ps < kIdxCap / kPass; ++ps) {
      const int i0 = ps * kPass + 4 * tid;
      if (i0 >= nblk * NKEY) continue;
      int r[4] = {raw[ps].x, raw[ps].y, raw[ps].z, raw[ps].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = r[e];
        const bool ok = (i0 + e < nslot) && t >= 0 && t < Lb;
        if (validate && i0 + e < nslot) {
          if (!ok && t != -1) atomicOr(a.status, 1u);
          if (ok) {
            const uint32_t bit = 1u << (t & 31);
            const uint32_t old = atomicOr(a.bitmap + (int64_t)b * a.bitmap_words + (t >> 5), bit);
            if (old & bit) atomicOr(a.status, 2u);
          }
        }
        r[e] = ok ? t : -1;
      }
      *reinterpret_cast<int4*>(sidx + i0) = make_int4(r[0], r[1], r[2], r[3]);
    }
  } else {
    load_query();
    if (validate) {
      for (int i = tid; i < nslot; i += 256) {
        const int t = s0 + i;
        if (t < Lb) atomicOr(a.bitmap + (int64_t)b * a.bitmap_words + (t >> 5), 1u << (t & 31));
      }
    }
  }
  __syncthreads();

  auto row_of = [&](int i) -> int {  // slot i of this split -> cache row or -1
    if constexpr (dense) {
      const int t = s0 + i;
      return (i < nslot && t < Lb) ? t : -1;
    }
    return sidx[i];
  };

  const uint32_t kv_rb = (uint32_t)(a.kv_st * 2), pe_rb = (uint32_t)(a.pe_st * 2);
  const i32x4 rkv = buffer_rsrc(a.kv + (int64_t)b * a.kv_sb, (uint32_t)Lb * kv_rb);
  const i32x4 rpe = buffer_rsrc(a.pe + (int64_t)b * a.pe_sb, (uint32_t)Lb * pe_rb);
  const uint32_t lds0 = (uint32_t)(uintptr_t)s3;

  // Gather block p into buffer p % NBUF.  Wave w moves key groups
  // (8 keys each) KL*w .. KL*w+KL-1, all 9 lines; lane l takes key
  // 8 * group + l / 8 and 16-byte position l % 8 of each line.
  auto issue = [&](int p) {
    const uint32_t dst0 = lds0 + (uint32_t)((p % NBUF) * BUF);
#pragma unroll
    for (int kg = 0; kg < KL; ++kg) {
      const int key = 8 * (KL * wave + kg) + (lane >> 3);
      const int row = row_of(p * NKEY + key);
      const uint32_t q16 = (((uint32_t)(lane & 7)) ^ seg_swz((uint32_t)key)) * 16u;
      const uint32_t okv = row >= 0 ? (uint32_t)row * kv_rb + q16 : kMaskedOffset;
      const uint32_t ope = row >= 0 ? (uint32_t)row * pe_rb + q16 : kMaskedOffset;
      const uint32_t dst = dst0 + (uint32_t)(8 * (KL * wave + kg)) * 128u;
#pragma unroll
      for (int m = 0; m < 8; ++m) dma16(rkv, dst + (uint32_t)(m * NKEY * 128), okv + (uint32_t)(m * 128));
      dma16(rpe, dst + (uint32_t)(8 * NKEY * 128), ope);
    }
  };

  f32x16 acc[16];
#pragma unroll
  for (int ct = 0; ct < 16; ++ct) acc[ct] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Per-lane LDS offsets.  Score reads: key kl*32 + lane%32, chunk
  // 2 st + hh (line st / 4, chunk-in-line 2 (st % 4) + hh).
  uint32_t qk_base[4];
  {
    const uint32_t key = (uint32_t)(kl * 32 + (lane & 31));
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      qk_base[s4] = key * 128u + (((uint32_t)(2 * s4 + hh)) ^ seg_swz(key)) * 16u;
  }
  // Transpose reads: source lane i of group g reads key
  // kl*32 + 16 ks + 8 r + 4 hh + i/4, columns 32 ct + 16 gm + 4 (i % 4):
  // chunk-in-line 4 (ct % 2) + 2 gm + (i % 4) / 2, byte 8 (i % 2).
  const int i16 = lane & 15, gm = (lane >> 4) & 1;
  uint32_t pc_base[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1) {
      const uint32_t key = (uint32_t)(kl * 32 + 8 * r + 4 * hh + (i16 >> 2));
      const uint32_t q = (uint32_t)(4 * c1 + 2 * gm + ((i16 & 3) >> 1));
      pc_base[r][c1] = key * 128u + ((q ^ seg_swz(key)) * 16u) + 8u * (uint32_t)(i16 & 1);
    }

#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < nblk) issue(p);

  for (int j = 0; j < nblk; ++j) {
    // Wait for block j: blocks j+1 .. j+NBUF-2 (when they exist) may stay in flight.
    const int after = min(NBUF - 2, nblk - 1 - j);
    if (NBUF >= 4 && after >= 2) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * GPW) : "memory");
    } else if (NBUF >= 3 && after >= 1) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(GPW) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (j + NBUF - 1 < nblk) issue(j + NBUF - 1);

    const char LDS_AS* buf = s3 + (j % NBUF) * BUF;

    // Scores for this wave's 32 keys and 32 heads.  LDS reads run QK_AHEAD
    // steps ahead of the MFMAs; the fences keep the scheduler from hoisting
    // more (the query operand and the accumulators hold 400 registers).
    f32x16 sacc = {};
    {
      constexpr int QK_AHEAD = 3;
      bf16x8 ring[QK_AHEAD + 1];
      auto qk_ld = [&](int st) {
        const uint32_t off = qk_base[st & 3] + (uint32_t)((st >> 2) * NKEY * 128);
        return *(const bf16x8 LDS_AS*)(buf + off);
      };
#pragma unroll
      for (int st = 0; st < QK_AHEAD; ++st) ring[st] = qk_ld(st);
#pragma unroll
      for (int st = 0; st < 36; ++st) {
        if (st + QK_AHEAD < 36) ring[(st + QK_AHEAD) % (QK_AHEAD + 1)] = qk_ld(st + QK_AHEAD);
        sacc = mfma32(ring[st % (QK_AHEAD + 1)], qf[st], sacc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    const bool v_ok = row_of(j * NKEY + kl * 32 + (lane & 31)) >= 0;
    const uint32_t vm = (uint32_t)__builtin_amdgcn_ballot_w64(v_ok);

    float t[16];
    float mloc = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kloc = 8 * (v >> 2) + 4 * hh + (v & 3);
      t[v] = ((vm >> kloc) & 1u) ? sacc[v] * a.scale_log2 : -INFINITY;
      mloc = fmaxf(mloc, t[v]);
    }
    if (a.flags & 2u) {
      float* so = a.scores + ((int64_t)b * kHeads + head) * a.k_max + s0 + j * NKEY + kl * 32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kloc = 8 * (v >> 2) + 4 * hh + (v & 3);
        if (j * NKEY + kl * 32 + kloc < nslot)
          so[kloc] = ((vm >> kloc) & 1u) ? sacc[v] * a.scale : -INFINITY;
      }
    }
    const float mblk = fmaxf(mloc, __shfl_xor(mloc, 32));
    const bool need = mblk > m_run + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float mnew = need ? mblk : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.f;
      l_run *= alpha;
      // acc *= alpha, on the accumulator registers in place: a plain C++
      // multiply would move all 256 accumulators into the VALU register file.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int ct = 0; ct < 16; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(acc[ct][v]), "=&v"(tmp)
                       : "v"(alpha));
        }
      asm volatile("s_nop 3" ::: "memory");
      m_run = mnew;
    }
    const float mref = (m_run == -INFINITY) ? 0.f : m_run;
    bf16x8 pb0, pb1;
    float lsum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = __builtin_amdgcn_exp2f(t[v] - mref);
      lsum += p;
      if (v < 8) pb0[v] = (__bf16)p;
      else pb1[v - 8] = (__bf16)p;
    }
    l_run += lsum;

    // Mix the latents of this block into the accumulators (transpose reads
    // PC_AHEAD MFMAs ahead, fenced as above).
    {
      constexpr int PC_AHEAD = 3;
      bf16x8 ring[PC_AHEAD + 1];
      auto pc_ld = [&](int i) {  // i = 2 ct + ks
        const int ct = i >> 1, ks = i & 1;
        const uint32_t o = (uint32_t)((ct >> 1) * NKEY * 128 + ks * 16 * 128);
        return tr_pair(buf + pc_base[0][ct & 1] + o, buf + pc_base[1][ct & 1] + o);
      };
#pragma unroll
      for (int i = 0; i < PC_AHEAD; ++i) ring[i] = pc_ld(i);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i + PC_AHEAD < 32) ring[(i + PC_AHEAD) % (PC_AHEAD + 1)] = pc_ld(i + PC_AHEAD);
        acc[i >> 1] = mfma32(ring[i % (PC_AHEAD + 1)], (i & 1) ? pb1 : pb0, acc[i >> 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  l_run += __shfl_xor(l_run, 32);

  if constexpr (KL == 2) {
    // Merge the two key lanes of each head slice through LDS.
    __syncthreads();
    float* mrg = reinterpret_cast<float*>(smem) + hs * (16 * 16 * 64 + 128);
    if (kl == 1) {
#pragma unroll
      for (int ct = 0; ct < 16; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) mrg[(ct * 16 + v) * 64 + lane] = acc[ct][v];
      mrg[16384 + lane] = m_run;
      mrg[16384 + 64 + lane] = l_run;
    }
    __syncthreads();
    if (kl == 0) {
      const float m2 = mrg[16384 + lane], l2 = mrg[16384 + 64 + lane];
      const float M = fmaxf(m_run, m2);
      const float a1 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
      const float a2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
      l_run = l_run * a1 + l2 * a2;
      m_run = M;
#pragma unroll
      for (int ct = 0; ct < 16; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[ct][v] = acc[ct][v] * a1 + mrg[(ct * 16 + v) * 64 + lane] * a2;
    }
  }
  if (kl != 0) return;

  if (a.S == 1) {
    const float inv = 1.0f / l_run;  // empty selection: 0 * inf = NaN
    uint16_t* o = a.o_latent + ((int64_t)b * kHeads + head) * kLatent + 4 * hh;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<uint2*>(o + 32 * ct + 8 * q4) =
            pack4(acc[ct][4 * q4] * inv, acc[ct][4 * q4 + 1] * inv, acc[ct][4 * q4 + 2] * inv,
                  acc[ct][4 * q4 + 3] * inv);
    if (a.lse != nullptr && hh == 0)
      a.lse[(int64_t)b * kHeads + head] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
    if (validate && hs == 0 && lane == 0 && !(l_run > 0.f)) atomicOr(a.status, 4u);
  } else {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;  // an empty split contributes nothing
    uint16_t* po = a.part_o + (((int64_t)s * a.B + b) * kHeads + head) * kLatent + 4 * hh;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<uint2*>(po + 32 * ct + 8 * q4) =
            pack4(acc[ct][4 * q4] * inv, acc[ct][4 * q4 + 1] * inv, acc[ct][4 * q4 + 2] * inv,
                  acc[ct][4 * q4 + 3] * inv);
    if (hh == 0) {
      float* pml = a.part_ml + (((int64_t)s * a.B + b) * kHeads + head) * 2;
      pml[0] = m_run;
      pml[1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// combine: O~ = sum_s g_s O~_s, g_s = 2^(m_s - M) l_s / L, L = sum_s 2^(m_s - M) l_s
// Workgroup = (sequence, 2 heads); each thread owns 4 latent columns.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  const int b = blockIdx.x >> 6;
  const int head = (blockIdx.x & 63) * 2 + (threadIdx.x >> 7);
  const int col = (threadIdx.x & 127) * 4;
  const int64_t stride_s = (int64_t)a.B * kHeads;
  const int64_t bh = (int64_t)b * kHeads + head;
  float M = -INFINITY;
  for (int s = 0; s < a.S; ++s) M = fmaxf(M, a.part_ml[(s * stride_s + bh) * 2]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.S; ++s) {
    const float ms = a.part_ml[(s * stride_s + bh) * 2];
    const float wl = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M) * a.part_ml[(s * stride_s + bh) * 2 + 1];
    L += wl;
    const uint2 v = *reinterpret_cast<const uint2*>(a.part_o + (s * stride_s + bh) * kLatent + col);
    acc[0] += wl * __uint_as_float(v.x << 16);
    acc[1] += wl * __uint_as_float(v.x & 0xffff0000u);
    acc[2] += wl * __uint_as_float(v.y << 16);
    acc[3] += wl * __uint_as_float(v.y & 0xffff0000u);
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
// fp8 dequantisation (one-time set-up).  E4M3FN from its definition: sign,
// 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal
// (m/8 * 2^-6); 0x7F / 0xFF are NaN.  The product with the fp32 block scale
// is rounded to bf16 from its exact value: p = fl(v * s) plus the exact
// residual fma(v, s, -p) decide the rare ties that fl() creates.
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
  hipLaunchKernelGGL(absorb_kernel, dim3(kHeads * 2), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_decode(const DecodeArgs& a, int head_groups, void* stream) {
  const int units = a.B * a.S;
  const int groups8 = (units + 7) / 8;
  const hipStream_t st = (hipStream_t)stream;
  const bool dense = a.indices == nullptr;
  if (head_groups == 2) {
    if (dense) hipLaunchKernelGGL((decode_kernel<2, 2, true>), dim3(groups8 * 16), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((decode_kernel<2, 2, false>), dim3(groups8 * 16), dim3(256), 0, st, a);
  } else {
    if (dense) hipLaunchKernelGGL((decode_kernel<1, 4, true>), dim3(groups8 * 8), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((decode_kernel<1, 4, false>), dim3(groups8 * 8), dim3(256), 0, st, a);
  }
  return (int)hipGetLastError();
}

int launch_combine(const CombineArgs& a, void* stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.B * 64), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_value_up(const ValueUpArgs& a, void* stream) {
  if (a.o_latent == nullptr)
    hipLaunchKernelGGL(value_up_kernel<true>, dim3(kHeads), dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(value_up_kernel<false>, dim3(kHeads), dim3(256), 0, (hipStream_t)stream, a);
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

}  // namespace mla
