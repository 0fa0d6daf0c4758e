// C-ABI entry points of libmla_decode: argument validation, launch planning
// and workspace sizing on the host, then one kernel launch per call.
// Nothing here includes HIP headers; kernels are reached through
// mla_kernels.h.  See include/mla_decode.h for the contract of each call.
#include "mla_decode.h"

#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "mla_kernels.h"

static_assert(MLA_MAX_SLOTS_PER_SPLIT == mla::kIdxCap, "index staging capacity");

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool stride8(int64_t s) { return s >= 0 && (s & 7) == 0; }

int hip_status(int err) {
  if (err == 0) return MLA_OK;
  g_last_hip_error = err;
  return MLA_ERR_HIP;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Head counts a call may take: all 128 heads, or one GPU's share of them
// when the heads are sharded across GPUs.
bool heads_ok(int32_t H) { return H == 16 || H == 32 || H == 64 || H == 128; }

// Index slots per split: ceil(k_max / S) rounded up to whole key blocks.
int64_t split_chunk(int32_t k_max, int32_t S) { return ceil_div(ceil_div(k_max, S), 32) * 32; }

}  // namespace

extern "C" {

int mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MLA_ERR_BAD_DIM: return "invalid size, split count or head-group count";
    case MLA_ERR_ALIGNMENT: return "pointer not 16-byte aligned or stride not a multiple of 8 elements";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than mla_workspace_bytes()";
    case MLA_ERR_UNSUPPORTED: return "stride smaller than the fixed row width, or a head count other than 16/32/64/128";
    case MLA_ERR_HIP: return "HIP runtime error (see mla_last_hip_error)";
    case MLA_ERR_RANGE: return "a sequence's cache or q_pe span exceeds 2 GiB";
    case MLA_ERR_SCRATCH_LIMIT: return "the split partials exceed the library's static scratch (mla_noalloc_scratch_bytes)";
    default: return "unknown status";
  }
}

int mla_last_hip_error(void) { return g_last_hip_error; }

size_t mla_workspace_bytes_heads(int32_t n_heads, int32_t B, int32_t num_splits) {
  if (!heads_ok(n_heads) || B < 1 || num_splits < 1 || num_splits > MLA_MAX_SPLITS) return 0;
  if (num_splits == 1) return 0;
  const size_t units = (size_t)num_splits * (size_t)B * n_heads;
  return units * MLA_LATENT_DIM * sizeof(uint16_t) + units * 2 * sizeof(float);
}

size_t mla_workspace_bytes(int32_t B, int32_t num_splits) { return mla_workspace_bytes_heads(MLA_HEADS, B, num_splits); }

// Cost model (in nanoseconds) over splits 1..64, one workgroup per CU:
//  * fixed: every round of workgroups loads its query tile and writes its
//    normalised mix, ~14 us;
//  * keys: ~68 ns per key slot of a split (a 32-key block of 68 MFMA
//    32x32x16 per wave plus its gather, measured ~2.2 us);
//  * partials: with S > 1 the mixes are re-read by the combine.
// Sparse mode caps a split at MLA_MAX_SLOTS_PER_SPLIT slots.
int mla_plan(int32_t B, int32_t k_max, int32_t dense, int32_t num_cus, int32_t* num_splits) {
  if (B < 1 || k_max < 1 || !num_splits) return MLA_ERR_BAD_DIM;
  if (num_cus <= 0) num_cus = 256;
  double best = 1e300;
  int bs = 0;
  for (int S = 1; S <= MLA_MAX_SPLITS; ++S) {
    const int64_t chunk = split_chunk(k_max, S);
    if (!dense && chunk > MLA_MAX_SLOTS_PER_SPLIT) continue;
    if (S > 1 && (int64_t)(S - 1) * chunk >= k_max) continue;  // an empty split (a larger S may fit again)
    const int64_t rounds = ceil_div((int64_t)B * S, num_cus);
    const double t_round = 14.0e3 + (double)chunk * 68.0;
    const double t_part = S > 1 ? (double)S * B * MLA_HEADS * MLA_LATENT_DIM * 2.0 / 5.0e3 : 0.0;
    const double t = (double)rounds * t_round + t_part;
    if (t < best * 0.999) {
      best = t;
      bs = S;
    }
  }
  if (bs == 0) return MLA_ERR_BAD_DIM;
  *num_splits = bs;
  return MLA_OK;
}

}  // extern "C"

namespace {

int absorb_impl(const void* q_nope, int64_t q_nope_sb, int64_t q_nope_sh, const void* wkv_b,
                const mla::Fp8Weight& fp8, void* q_abs, int32_t B, void* stream, int32_t H = MLA_HEADS) {
  if (!heads_ok(H)) return MLA_ERR_UNSUPPORTED;
  if (!q_nope || !q_abs || (!wkv_b && !fp8.w_fp8)) return MLA_ERR_NULL_POINTER;
  if (B < 1 || B > 65536) return MLA_ERR_BAD_DIM;
  if (!aligned16(q_nope) || !aligned16(q_abs) || !stride8(q_nope_sb) || !stride8(q_nope_sh) ||
      (wkv_b && !aligned16(wkv_b)))
    return MLA_ERR_ALIGNMENT;
  // One head's rows are read with 32-bit byte offsets.
  if (q_nope_sb < 0 || q_nope_sh < 0 || ((int64_t)(B - 1) * q_nope_sb + MLA_NOPE_DIM) * 2 > (int64_t)UINT32_MAX)
    return MLA_ERR_RANGE;
  mla::AbsorbArgs a = {};
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_sb = q_nope_sb;
  a.q_sh = q_nope_sh;
  a.wkv_b = static_cast<const uint16_t*>(wkv_b);
  a.q_abs = static_cast<uint16_t*>(q_abs);
  a.B = B;
  a.H = H;
  a.fp8 = fp8;
  return hip_status(mla::launch_absorb(a, stream));
}

// The fp8 weight arguments: codes 16-byte aligned, scales 4-byte aligned,
// the optional formed-weight output 16-byte aligned.
int fp8_weight(const void* w_fp8, const float* w_scale, void* w_formed, mla::Fp8Weight* out) {
  if (!w_fp8 || !w_scale) return MLA_ERR_NULL_POINTER;
  if (!aligned16(w_fp8) || (reinterpret_cast<uintptr_t>(w_scale) & 3u) || (w_formed && !aligned16(w_formed)))
    return MLA_ERR_ALIGNMENT;
  out->w_fp8 = static_cast<const uint8_t*>(w_fp8);
  out->w_scale = w_scale;
  out->w_formed = static_cast<uint16_t*>(w_formed);
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_absorb_q(const void* q_nope, int64_t q_nope_sb, int64_t q_nope_sh,
                 const void* wkv_b, void* q_abs, int32_t B, void* stream) {
  if (!wkv_b) return MLA_ERR_NULL_POINTER;
  return absorb_impl(q_nope, q_nope_sb, q_nope_sh, wkv_b, mla::Fp8Weight{}, q_abs, B, stream);
}

int mla_absorb_q_heads(int32_t n_heads, const void* q_nope, int64_t q_nope_sb, int64_t q_nope_sh,
                       const void* wkv_b, void* q_abs, int32_t B, void* stream) {
  if (!wkv_b) return MLA_ERR_NULL_POINTER;
  return absorb_impl(q_nope, q_nope_sb, q_nope_sh, wkv_b, mla::Fp8Weight{}, q_abs, B, stream, n_heads);
}

int mla_absorb_q_fp8(const void* q_nope, int64_t q_nope_sb, int64_t q_nope_sh, const void* w_fp8,
                     const float* w_scale, void* q_abs, int32_t B, void* w_formed, void* stream) {
  mla::Fp8Weight f;
  const int st = fp8_weight(w_fp8, w_scale, w_formed, &f);
  if (st != MLA_OK) return st;
  return absorb_impl(q_nope, q_nope_sb, q_nope_sh, nullptr, f, q_abs, B, stream);
}

}  // extern "C"

namespace {

// Argument checks and kernel arguments of mla_sparse_decode (shared with the
// allocation-free variant, which passes its static scratch as the workspace).
int prepare_decode(const void* q_abs, const void* q_pe, int64_t q_pe_sb, int64_t q_pe_sh,
                   const void* kv, int64_t kv_sb, int64_t kv_st,
                   const void* pe, int64_t pe_sb, int64_t pe_st,
                   const int32_t* seq_lens, int32_t max_len,
                   const int32_t* indices, int32_t k_max, float scale, int32_t B,
                   int32_t num_splits, void* workspace, size_t ws_bytes,
                   void* o_latent, float* lse,
                   uint32_t flags, uint32_t* attended_bitmap, int64_t bitmap_words,
                   float* scores_out, uint32_t* status_dev, mla::DecodeArgs* out,
                   int32_t prefill_T = 0, int32_t H = MLA_HEADS) {
  if (!heads_ok(H)) return MLA_ERR_UNSUPPORTED;
  // prefill_T > 0: prefill rows (B = prompts * prefill_T, token r % T of
  // prompt r / T, causal lengths, no seq_lens, max_len = T).
  if (!q_abs || !q_pe || !kv || !pe || (!seq_lens && prefill_T == 0)) return MLA_ERR_NULL_POINTER;
  if (B < 1 || B > 65536 || k_max < 1 || max_len < 1) return MLA_ERR_BAD_DIM;
  if (num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_BAD_DIM;
  if (!indices && k_max < max_len) return MLA_ERR_BAD_DIM;
  const int64_t chunk = split_chunk(k_max, num_splits);
  if (indices && chunk > MLA_MAX_SLOTS_PER_SPLIT) return MLA_ERR_BAD_DIM;
  if ((int64_t)B * num_splits > (int64_t)1 << 30) return MLA_ERR_BAD_DIM;
  if (!aligned16(q_abs) || !aligned16(q_pe) || !aligned16(kv) || !aligned16(pe) ||
      !stride8(q_pe_sb) || !stride8(q_pe_sh) || !stride8(kv_sb) || !stride8(kv_st) ||
      !stride8(pe_sb) || !stride8(pe_st))
    return MLA_ERR_ALIGNMENT;
  if (kv_st < MLA_LATENT_DIM || pe_st < MLA_ROPE_DIM) return MLA_ERR_UNSUPPORTED;
  const int64_t span_limit = ((int64_t)1 << 31) - 1;
  if ((int64_t)max_len * kv_st * 2 > span_limit || (int64_t)max_len * pe_st * 2 > span_limit ||
      ((int64_t)(H - 1) * q_pe_sh + MLA_ROPE_DIM) * 2 > span_limit)
    return MLA_ERR_RANGE;
  if (num_splits == 1) {
    if (!o_latent) return MLA_ERR_NULL_POINTER;
    if (!aligned16(o_latent)) return MLA_ERR_ALIGNMENT;
  } else {
    if (!workspace) return MLA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return MLA_ERR_ALIGNMENT;
    if (ws_bytes < mla_workspace_bytes_heads(H, B, num_splits)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  }
  if (flags & MLA_FLAG_VALIDATE) {
    if (!status_dev || !attended_bitmap) return MLA_ERR_NULL_POINTER;
    if (bitmap_words < ceil_div(max_len, 32)) return MLA_ERR_BAD_DIM;
  }
  if ((flags & MLA_FLAG_WRITE_SCORES) && !scores_out) return MLA_ERR_NULL_POINTER;

  mla::DecodeArgs& a = *out;
  a.q_abs = static_cast<const uint16_t*>(q_abs);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.q_pe_sb = q_pe_sb;
  a.q_pe_sh = q_pe_sh;
  a.kv = static_cast<const uint16_t*>(kv);
  a.kv_sb = kv_sb;
  a.kv_st = kv_st;
  a.pe = static_cast<const uint16_t*>(pe);
  a.pe_sb = pe_sb;
  a.pe_st = pe_st;
  a.seq_lens = seq_lens;
  a.indices = indices;
  a.max_len = max_len;
  a.k_max = k_max;
  a.chunk = (int32_t)chunk;
  a.B = B;
  a.H = H;
  a.S = num_splits;
  a.causal = prefill_T > 0 ? 1 : 0;
  a.rows_per_seq = prefill_T > 0 ? prefill_T : 1;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  const size_t units = (size_t)num_splits * (size_t)B * H;
  a.part_o = num_splits > 1 ? static_cast<uint16_t*>(workspace) : nullptr;
  a.part_ml = num_splits > 1
                  ? reinterpret_cast<float*>(static_cast<uint16_t*>(workspace) + units * MLA_LATENT_DIM)
                  : nullptr;
  a.o_latent = static_cast<uint16_t*>(o_latent);
  a.lse = lse;
  a.flags = flags;
  a.bitmap = attended_bitmap;
  a.bitmap_words = bitmap_words;
  a.scores = scores_out;
  a.status = status_dev;
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_sparse_decode_heads(int32_t n_heads, const void* q_abs, const void* q_pe, int64_t q_pe_sb, int64_t q_pe_sh,
                            const void* kv, int64_t kv_sb, int64_t kv_st,
                            const void* pe, int64_t pe_sb, int64_t pe_st,
                            const int32_t* seq_lens, int32_t max_len,
                            const int32_t* indices, int32_t k_max, float scale, int32_t B,
                            int32_t num_splits, void* workspace, size_t ws_bytes,
                            void* o_latent, float* lse,
                            uint32_t flags, uint32_t* attended_bitmap, int64_t bitmap_words,
                            float* scores_out, uint32_t* status_dev, void* stream) {
  mla::DecodeArgs a;
  const int st = prepare_decode(q_abs, q_pe, q_pe_sb, q_pe_sh, kv, kv_sb, kv_st, pe, pe_sb, pe_st, seq_lens,
                                max_len, indices, k_max, scale, B, num_splits, workspace, ws_bytes, o_latent, lse,
                                flags, attended_bitmap, bitmap_words, scores_out, status_dev, &a, 0, n_heads);
  if (st != MLA_OK) return st;
  return hip_status(mla::launch_decode(a, stream));
}

int mla_sparse_decode(const void* q_abs, const void* q_pe, int64_t q_pe_sb, int64_t q_pe_sh,
                      const void* kv, int64_t kv_sb, int64_t kv_st,
                      const void* pe, int64_t pe_sb, int64_t pe_st,
                      const int32_t* seq_lens, int32_t max_len,
                      const int32_t* indices, int32_t k_max, float scale, int32_t B,
                      int32_t num_splits, void* workspace, size_t ws_bytes,
                      void* o_latent, float* lse,
                      uint32_t flags, uint32_t* attended_bitmap, int64_t bitmap_words,
                      float* scores_out, uint32_t* status_dev, void* stream) {
  return mla_sparse_decode_heads(MLA_HEADS, q_abs, q_pe, q_pe_sb, q_pe_sh, kv, kv_sb, kv_st, pe, pe_sb, pe_st,
                                 seq_lens, max_len, indices, k_max, scale, B, num_splits, workspace, ws_bytes,
                                 o_latent, lse, flags, attended_bitmap, bitmap_words, scores_out, status_dev, stream);
}

size_t mla_noalloc_scratch_bytes(void) { return mla::kScratchBytes; }

int mla_sparse_decode_noalloc(const void* q_abs, const void* q_pe, int64_t q_pe_sb, int64_t q_pe_sh,
                              const void* kv, int64_t kv_sb, int64_t kv_st,
                              const void* pe, int64_t pe_sb, int64_t pe_st,
                              const int32_t* seq_lens, int32_t max_len,
                              const int32_t* indices, int32_t k_max, float scale, int32_t B,
                              int32_t num_splits, void* o_latent, float* lse,
                              uint32_t flags, uint32_t* attended_bitmap, int64_t bitmap_words,
                              float* scores_out, uint32_t* status_dev, void* stream) {
  if (B >= 1 && num_splits > 1 && num_splits <= MLA_MAX_SPLITS &&
      mla_workspace_bytes(B, num_splits) > mla::kScratchBytes)
    return MLA_ERR_SCRATCH_LIMIT;
  // Every argument is checked before the scratch address is looked up (the
  // placeholder stands for the scratch, which is aligned and large enough);
  // the partials' pointers are set from the real address after.
  void* const placeholder = reinterpret_cast<void*>(uintptr_t{256});
  mla::DecodeArgs a;
  const int st = prepare_decode(q_abs, q_pe, q_pe_sb, q_pe_sh, kv, kv_sb, kv_st, pe, pe_sb, pe_st, seq_lens,
                                max_len, indices, k_max, scale, B, num_splits, placeholder, mla::kScratchBytes,
                                o_latent, lse, flags, attended_bitmap, bitmap_words, scores_out, status_dev, &a);
  if (st != MLA_OK) return st;
  if (num_splits > 1 && !o_latent) return MLA_ERR_NULL_POINTER;
  if (num_splits > 1 && !aligned16(o_latent)) return MLA_ERR_ALIGNMENT;
  if (num_splits > 1) {
    void* ws = nullptr;
    const int e = mla::scratch_buffer(&ws);
    if (e != 0) return hip_status(e);
    const size_t units = (size_t)num_splits * (size_t)B * MLA_HEADS;
    a.part_o = static_cast<uint16_t*>(ws);
    a.part_ml = reinterpret_cast<float*>(static_cast<uint16_t*>(ws) + units * MLA_LATENT_DIM);
  }
  int r = hip_status(mla::launch_decode(a, stream));
  if (r != MLA_OK || num_splits == 1) return r;
  mla::CombineArgs c;
  c.part_o = a.part_o;
  c.part_ml = a.part_ml;
  c.B = B;
  c.S = num_splits;
  c.H = MLA_HEADS;
  c.o_latent = static_cast<uint16_t*>(o_latent);
  c.lse = lse;
  c.status = (flags & MLA_FLAG_VALIDATE) ? status_dev : nullptr;
  return hip_status(mla::launch_combine(c, stream));
}

size_t mla_prefill_workspace_bytes(int32_t B, int32_t T, int32_t num_splits) {
  if (B < 1 || T < 1 || (int64_t)B * T > 65536) return 0;
  const int32_t rows = B * T;
  const size_t tile = (size_t)rows * MLA_HEADS * MLA_LATENT_DIM * sizeof(uint16_t);
  if (num_splits == 1) return 2 * tile;
  const size_t part = mla_workspace_bytes(rows, num_splits);
  return part == 0 ? 0 : tile + part;
}

int mla_sparse_prefill(const void* q_nope, int64_t q_nope_st, int64_t q_nope_sh,
                       const void* q_pe, int64_t q_pe_st, int64_t q_pe_sh,
                       const void* kv, int64_t kv_sb, int64_t kv_st,
                       const void* pe, int64_t pe_sb, int64_t pe_st,
                       const void* wkv_b, const int32_t* indices, int32_t k_max, float scale,
                       int32_t B, int32_t T, int32_t num_splits, void* workspace, size_t ws_bytes,
                       void* out, int64_t out_st, int64_t out_sh, float* lse,
                       uint32_t flags, uint32_t* attended_bitmap, int64_t bitmap_words,
                       uint32_t* status_dev, void* stream) {
  if (!q_nope || !wkv_b || !out || !workspace) return MLA_ERR_NULL_POINTER;
  if (B < 1 || T < 1 || (int64_t)B * T > 65536) return MLA_ERR_BAD_DIM;
  if (flags & MLA_FLAG_WRITE_SCORES) return MLA_ERR_BAD_DIM;  // not offered for prefill
  if (!indices && k_max < T) return MLA_ERR_BAD_DIM;
  if (!aligned16(q_nope) || !aligned16(wkv_b) || !aligned16(out) || !aligned16(workspace) ||
      !stride8(q_nope_st) || !stride8(q_nope_sh) || !stride8(out_st) || !stride8(out_sh))
    return MLA_ERR_ALIGNMENT;
  const int32_t rows = B * T;
  if (num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_BAD_DIM;
  if (ws_bytes < mla_prefill_workspace_bytes(B, T, num_splits)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (((int64_t)(rows - 1) * q_nope_st + MLA_NOPE_DIM) * 2 > (int64_t)UINT32_MAX) return MLA_ERR_RANGE;
  const size_t tile = (size_t)rows * MLA_HEADS * MLA_LATENT_DIM * sizeof(uint16_t);
  void* q_abs = workspace;
  void* rest = static_cast<char*>(workspace) + tile;
  mla::DecodeArgs d;
  int st = prepare_decode(q_abs, q_pe, q_pe_st, q_pe_sh, kv, kv_sb, kv_st, pe, pe_sb, pe_st, nullptr, T,
                          indices, k_max, scale, rows, num_splits, rest, ws_bytes - tile,
                          num_splits == 1 ? rest : nullptr, lse, flags, attended_bitmap, bitmap_words, nullptr,
                          status_dev, &d, T);
  if (st != MLA_OK) return st;
  if ((int64_t)num_splits * rows * MLA_HEADS * 8 > (int64_t)INT32_MAX) return MLA_ERR_RANGE;
  mla::AbsorbArgs ab = {};
  ab.q_nope = static_cast<const uint16_t*>(q_nope);
  ab.q_sb = q_nope_st;
  ab.q_sh = q_nope_sh;
  ab.wkv_b = static_cast<const uint16_t*>(wkv_b);
  ab.q_abs = static_cast<uint16_t*>(q_abs);
  ab.B = rows;
  ab.H = MLA_HEADS;
  st = hip_status(mla::launch_absorb(ab, stream));
  if (st != MLA_OK) return st;
  st = hip_status(mla::launch_decode(d, stream));
  if (st != MLA_OK) return st;
  mla::ValueUpArgs v = {};
  v.wkv_b = static_cast<const uint16_t*>(wkv_b);
  v.out = static_cast<uint16_t*>(out);
  v.out_sb = out_st;
  v.out_sh = out_sh;
  v.B = rows;
  v.H = MLA_HEADS;
  if (num_splits == 1) {
    v.o_latent = static_cast<const uint16_t*>(rest);
  } else {
    v.o_latent = nullptr;
    v.part_o = d.part_o;
    v.part_ml = d.part_ml;
    v.S = num_splits;
    v.lse = lse;
    v.status = (flags & MLA_FLAG_VALIDATE) ? status_dev : nullptr;
  }
  return hip_status(mla::launch_value_up(v, stream));
}

int mla_combine_heads(int32_t n_heads, const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                      void* o_latent, float* lse, uint32_t* status_dev, void* stream) {
  if (!heads_ok(n_heads)) return MLA_ERR_UNSUPPORTED;
  if (B < 1 || B > 65536 || num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_BAD_DIM;
  if (num_splits == 1) return MLA_OK;
  if (!workspace || !o_latent) return MLA_ERR_NULL_POINTER;
  if (!aligned16(workspace) || !aligned16(o_latent)) return MLA_ERR_ALIGNMENT;
  if (ws_bytes < mla_workspace_bytes_heads(n_heads, B, num_splits)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  const size_t units = (size_t)num_splits * (size_t)B * n_heads;
  mla::CombineArgs a;
  a.part_o = static_cast<const uint16_t*>(workspace);
  a.part_ml = reinterpret_cast<const float*>(static_cast<const uint16_t*>(workspace) + units * MLA_LATENT_DIM);
  a.B = B;
  a.S = num_splits;
  a.H = n_heads;
  a.o_latent = static_cast<uint16_t*>(o_latent);
  a.lse = lse;
  a.status = status_dev;
  return hip_status(mla::launch_combine(a, stream));
}

int mla_combine(const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                void* o_latent, float* lse, uint32_t* status_dev, void* stream) {
  return mla_combine_heads(MLA_HEADS, workspace, ws_bytes, B, num_splits, o_latent, lse, status_dev, stream);
}

}  // extern "C"

namespace {

int value_up_impl(const void* o_latent, const void* wkv_b, const mla::Fp8Weight& fp8, void* out,
                  int64_t out_sb, int64_t out_sh, int32_t B, void* stream, int32_t H = MLA_HEADS) {
  if (!heads_ok(H)) return MLA_ERR_UNSUPPORTED;
  if (!o_latent || !out || (!wkv_b && !fp8.w_fp8)) return MLA_ERR_NULL_POINTER;
  if (B < 1 || B > 65536) return MLA_ERR_BAD_DIM;
  if (!aligned16(o_latent) || (wkv_b && !aligned16(wkv_b)) || !aligned16(out) || !stride8(out_sb) ||
      !stride8(out_sh))
    return MLA_ERR_ALIGNMENT;
  mla::ValueUpArgs a = {};
  a.o_latent = static_cast<const uint16_t*>(o_latent);
  a.wkv_b = static_cast<const uint16_t*>(wkv_b);
  a.out = static_cast<uint16_t*>(out);
  a.out_sb = out_sb;
  a.out_sh = out_sh;
  a.B = B;
  a.H = H;
  a.fp8 = fp8;
  return hip_status(mla::launch_value_up(a, stream));
}

int combine_value_up_impl(const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                          const void* wkv_b, const mla::Fp8Weight& fp8, void* out, int64_t out_sb, int64_t out_sh,
                          float* lse, uint32_t* status_dev, void* stream, int32_t H = MLA_HEADS) {
  if (!heads_ok(H)) return MLA_ERR_UNSUPPORTED;
  if (B < 1 || B > 65536 || num_splits < 2 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_BAD_DIM;
  if (!workspace || !out || (!wkv_b && !fp8.w_fp8)) return MLA_ERR_NULL_POINTER;
  if (!aligned16(workspace) || (wkv_b && !aligned16(wkv_b)) || !aligned16(out) || !stride8(out_sb) ||
      !stride8(out_sh))
    return MLA_ERR_ALIGNMENT;
  if (ws_bytes < mla_workspace_bytes_heads(H, B, num_splits)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  const size_t units = (size_t)num_splits * (size_t)B * H;
  if (units * 8 > (size_t)INT32_MAX) return MLA_ERR_RANGE;  // (max, sum) addressed with 32-bit offsets
  mla::ValueUpArgs a = {};
  a.o_latent = nullptr;
  a.wkv_b = static_cast<const uint16_t*>(wkv_b);
  a.out = static_cast<uint16_t*>(out);
  a.out_sb = out_sb;
  a.out_sh = out_sh;
  a.B = B;
  a.part_o = static_cast<const uint16_t*>(workspace);
  a.part_ml = reinterpret_cast<const float*>(static_cast<const uint16_t*>(workspace) + units * MLA_LATENT_DIM);
  a.S = num_splits;
  a.H = H;
  a.lse = lse;
  a.status = status_dev;
  a.fp8 = fp8;
  return hip_status(mla::launch_value_up(a, stream));
}

}  // namespace

extern "C" {

int mla_value_up(const void* o_latent, const void* wkv_b, void* out,
                 int64_t out_sb, int64_t out_sh, int32_t B, void* stream) {
  if (!wkv_b) return MLA_ERR_NULL_POINTER;
  return value_up_impl(o_latent, wkv_b, mla::Fp8Weight{}, out, out_sb, out_sh, B, stream);
}

int mla_value_up_heads(int32_t n_heads, const void* o_latent, const void* wkv_b, void* out, int64_t out_sb,
                       int64_t out_sh, int32_t B, void* stream) {
  if (!wkv_b) return MLA_ERR_NULL_POINTER;
  return value_up_impl(o_latent, wkv_b, mla::Fp8Weight{}, out, out_sb, out_sh, B, stream, n_heads);
}

int mla_value_up_fp8(const void* o_latent, const void* w_fp8, const float* w_scale, void* out,
                     int64_t out_sb, int64_t out_sh, int32_t B, void* w_formed, void* stream) {
  mla::Fp8Weight f;
  const int st = fp8_weight(w_fp8, w_scale, w_formed, &f);
  if (st != MLA_OK) return st;
  return value_up_impl(o_latent, nullptr, f, out, out_sb, out_sh, B, stream);
}

static int output_proj_impl(const void* x, int64_t x_sb, const void* wo, bool packed, void* out, int64_t out_sb,
                            int32_t B, void* stream) {
  if (!x || !wo || !out) return MLA_ERR_NULL_POINTER;
  if (B < 1 || B > 65536 || x_sb < mla::kWoIn || out_sb < mla::kWoOut) return MLA_ERR_BAD_DIM;
  if (!aligned16(x) || !aligned16(wo) || !stride8(x_sb) || (reinterpret_cast<uintptr_t>(out) & 1u) != 0)
    return MLA_ERR_ALIGNMENT;
  // The rows of one launch (up to 64) are read with 32-bit byte offsets.
  if ((63 * x_sb + mla::kWoIn) * 2 > (int64_t)UINT32_MAX) return MLA_ERR_RANGE;
  for (int32_t b0 = 0; b0 < B; b0 += 64) {
    mla::OutProjArgs a;
    a.x = static_cast<const uint16_t*>(x) + (int64_t)b0 * x_sb;
    a.wo = static_cast<const uint16_t*>(wo);
    a.out = static_cast<uint16_t*>(out) + (int64_t)b0 * out_sb;
    a.x_sb = x_sb;
    a.out_sb = out_sb;
    a.B = B - b0 < 64 ? B - b0 : 64;
    a.packed = packed;
    a.part = nullptr;
    const int st = hip_status(mla::launch_output_proj(a, stream));
    if (st != MLA_OK) return st;
  }
  return MLA_OK;
}

int mla_output_proj(const void* x, int64_t x_sb, const void* wo, void* out, int64_t out_sb, int32_t B,
                    void* stream) {
  return output_proj_impl(x, x_sb, wo, false, out, out_sb, B, stream);
}

size_t mla_output_proj_split_workspace_bytes(int32_t B) {
  if (B < 1 || B > 65536) return 0;
  const int64_t rows = B < 64 ? B : 64;  // one launch's rows; larger batches reuse it launch after launch
  return (size_t)(mla::kOpSplit * rows * mla::kWoOut) * sizeof(float);
}

int mla_output_proj_split(const void* x, int64_t x_sb, const void* wo, void* out, int64_t out_sb, int32_t B,
                          void* workspace, size_t ws_bytes, void* stream) {
  if (!x || !wo || !out || !workspace) return MLA_ERR_NULL_POINTER;
  if (B < 1 || B > 65536 || x_sb < mla::kWoIn || out_sb < mla::kWoOut) return MLA_ERR_BAD_DIM;
  if (!aligned16(x) || !aligned16(wo) || !stride8(x_sb) || (reinterpret_cast<uintptr_t>(out) & 1u) != 0 ||
      !aligned16(workspace))
    return MLA_ERR_ALIGNMENT;
  if (ws_bytes < mla_output_proj_split_workspace_bytes(B)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if ((63 * x_sb + mla::kWoIn) * 2 > (int64_t)UINT32_MAX) return MLA_ERR_RANGE;
  for (int32_t b0 = 0; b0 < B; b0 += 64) {
    mla::OutProjArgs a;
    a.x = static_cast<const uint16_t*>(x) + (int64_t)b0 * x_sb;
    a.wo = static_cast<const uint16_t*>(wo);
    a.out = static_cast<uint16_t*>(out) + (int64_t)b0 * out_sb;
    a.x_sb = x_sb;
    a.out_sb = out_sb;
    a.B = B - b0 < 64 ? B - b0 : 64;
    a.packed = false;
    a.part = static_cast<float*>(workspace);
    const int st = hip_status(mla::launch_output_proj_split(a, stream));
    if (st != MLA_OK) return st;
  }
  return MLA_OK;
}

int mla_output_proj_pack(const void* wo, void* wo_packed, void* stream) {
  if (!wo || !wo_packed) return MLA_ERR_NULL_POINTER;
  if (!aligned16(wo) || !aligned16(wo_packed)) return MLA_ERR_ALIGNMENT;
  return hip_status(mla::launch_output_proj_pack(static_cast<const uint16_t*>(wo),
                                                 static_cast<uint16_t*>(wo_packed), stream));
}

int mla_output_proj_packed(const void* x, int64_t x_sb, const void* wo_packed, void* out, int64_t out_sb,
                           int32_t B, void* stream) {
  return output_proj_impl(x, x_sb, wo_packed, true, out, out_sb, B, stream);
}

int mla_combine_value_up(const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                         const void* wkv_b, void* out, int64_t out_sb, int64_t out_sh, float* lse,
                         uint32_t* status_dev, void* stream) {
  if (!wkv_b) return MLA_ERR_NULL_POINTER;
  return combine_value_up_impl(workspace, ws_bytes, B, num_splits, wkv_b, mla::Fp8Weight{}, out, out_sb, out_sh,
                               lse, status_dev, stream);
}

int mla_combine_value_up_heads(int32_t n_heads, const void* workspace, size_t ws_bytes, int32_t B,
                               int32_t num_splits, const void* wkv_b, void* out, int64_t out_sb, int64_t out_sh,
                               float* lse, uint32_t* status_dev, void* stream) {
  if (!wkv_b) return MLA_ERR_NULL_POINTER;
  return combine_value_up_impl(workspace, ws_bytes, B, num_splits, wkv_b, mla::Fp8Weight{}, out, out_sb, out_sh,
                               lse, status_dev, stream, n_heads);
}

int mla_combine_value_up_fp8(const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                             const void* w_fp8, const float* w_scale, void* out, int64_t out_sb, int64_t out_sh,
                             float* lse, uint32_t* status_dev, void* stream) {
  mla::Fp8Weight f;
  const int st = fp8_weight(w_fp8, w_scale, nullptr, &f);
  if (st != MLA_OK) return st;
  return combine_value_up_impl(workspace, ws_bytes, B, num_splits, nullptr, f, out, out_sb, out_sh, lse, status_dev,
                               stream);
}

int mla_dequant_wkv_b_fp8(const void* w_fp8, const float* scales, void* w_bf16, void* stream) {
  if (!w_fp8 || !scales || !w_bf16) return MLA_ERR_NULL_POINTER;
  if (!aligned16(w_fp8) || !aligned16(w_bf16) || (reinterpret_cast<uintptr_t>(scales) & 3u))
    return MLA_ERR_ALIGNMENT;
  mla::DequantArgs a;
  a.w = static_cast<const uint8_t*>(w_fp8);
  a.scales = scales;
  a.out = static_cast<uint16_t*>(w_bf16);
  return hip_status(mla::launch_dequant(a, stream));
}

}  // extern "C"
