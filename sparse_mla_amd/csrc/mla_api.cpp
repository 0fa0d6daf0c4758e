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
    case MLA_ERR_UNSUPPORTED: return "stride smaller than the fixed row width";
    case MLA_ERR_HIP: return "HIP runtime error (see mla_last_hip_error)";
    case MLA_ERR_RANGE: return "a sequence's cache or q_pe span exceeds 2 GiB";
    default: return "unknown status";
  }
}

int mla_last_hip_error(void) { return g_last_hip_error; }

size_t mla_workspace_bytes(int32_t B, int32_t num_splits) {
  if (B < 1 || num_splits < 1 || num_splits > MLA_MAX_SPLITS) return 0;
  if (num_splits == 1) return 0;
  const size_t units = (size_t)num_splits * (size_t)B * MLA_HEADS;
  return units * MLA_LATENT_DIM * sizeof(uint16_t) + units * 2 * sizeof(float);
}

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

int mla_absorb_q(const void* q_nope, int64_t q_nope_sb, int64_t q_nope_sh,
                 const void* wkv_b, void* q_abs, int32_t B, void* stream) {
  if (!q_nope || !wkv_b || !q_abs) return MLA_ERR_NULL_POINTER;
  if (B < 1 || B > 65536) return MLA_ERR_BAD_DIM;
  if (!aligned16(q_nope) || !aligned16(wkv_b) || !aligned16(q_abs) || !stride8(q_nope_sb) ||
      !stride8(q_nope_sh))
    return MLA_ERR_ALIGNMENT;
  // One head's rows are read with 32-bit byte offsets.
  if (q_nope_sb < 0 || q_nope_sh < 0 || ((int64_t)(B - 1) * q_nope_sb + MLA_NOPE_DIM) * 2 > (int64_t)UINT32_MAX)
    return MLA_ERR_RANGE;
  mla::AbsorbArgs a;
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_sb = q_nope_sb;
  a.q_sh = q_nope_sh;
  a.wkv_b = static_cast<const uint16_t*>(wkv_b);
  a.q_abs = static_cast<uint16_t*>(q_abs);
  a.B = B;
  return hip_status(mla::launch_absorb(a, stream));
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
  if (!q_abs || !q_pe || !kv || !pe || !seq_lens) return MLA_ERR_NULL_POINTER;
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
      ((int64_t)(MLA_HEADS - 1) * q_pe_sh + MLA_ROPE_DIM) * 2 > span_limit)
    return MLA_ERR_RANGE;
  if (num_splits == 1) {
    if (!o_latent) return MLA_ERR_NULL_POINTER;
    if (!aligned16(o_latent)) return MLA_ERR_ALIGNMENT;
  } else {
    if (!workspace) return MLA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return MLA_ERR_ALIGNMENT;
    if (ws_bytes < mla_workspace_bytes(B, num_splits)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  }
  if (flags & MLA_FLAG_VALIDATE) {
    if (!status_dev || !attended_bitmap) return MLA_ERR_NULL_POINTER;
    if (bitmap_words < ceil_div(max_len, 32)) return MLA_ERR_BAD_DIM;
  }
  if ((flags & MLA_FLAG_WRITE_SCORES) && !scores_out) return MLA_ERR_NULL_POINTER;

  mla::DecodeArgs a;
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
  a.S = num_splits;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  const size_t units = (size_t)num_splits * (size_t)B * MLA_HEADS;
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
  return hip_status(mla::launch_decode(a, stream));
}

int mla_combine(const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                void* o_latent, float* lse, uint32_t* status_dev, void* stream) {
  if (B < 1 || B > 65536 || num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_BAD_DIM;
  if (num_splits == 1) return MLA_OK;
  if (!workspace || !o_latent) return MLA_ERR_NULL_POINTER;
  if (!aligned16(workspace) || !aligned16(o_latent)) return MLA_ERR_ALIGNMENT;
  if (ws_bytes < mla_workspace_bytes(B, num_splits)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  const size_t units = (size_t)num_splits * (size_t)B * MLA_HEADS;
  mla::CombineArgs a;
  a.part_o = static_cast<const uint16_t*>(workspace);
  a.part_ml = reinterpret_cast<const float*>(static_cast<const uint16_t*>(workspace) + units * MLA_LATENT_DIM);
  a.B = B;
  a.S = num_splits;
  a.o_latent = static_cast<uint16_t*>(o_latent);
  a.lse = lse;
  a.status = status_dev;
  return hip_status(mla::launch_combine(a, stream));
}

int mla_value_up(const void* o_latent, const void* wkv_b, void* out,
                 int64_t out_sb, int64_t out_sh, int32_t B, void* stream) {
  if (!o_latent || !wkv_b || !out) return MLA_ERR_NULL_POINTER;
  if (B < 1 || B > 65536) return MLA_ERR_BAD_DIM;
  if (!aligned16(o_latent) || !aligned16(wkv_b) || !aligned16(out) || !stride8(out_sb) ||
      !stride8(out_sh))
    return MLA_ERR_ALIGNMENT;
  mla::ValueUpArgs a = {};
  a.o_latent = static_cast<const uint16_t*>(o_latent);
  a.wkv_b = static_cast<const uint16_t*>(wkv_b);
  a.out = static_cast<uint16_t*>(out);
  a.out_sb = out_sb;
  a.out_sh = out_sh;
  a.B = B;
  return hip_status(mla::launch_value_up(a, stream));
}

int mla_output_proj(const void* x, int64_t x_sb, const void* wo, void* out, int64_t out_sb, int32_t B,
                    void* stream) {
  if (!x || !wo || !out) return MLA_ERR_NULL_POINTER;
  if (B < 1 || B > 65536 || x_sb < mla::kWoIn || out_sb < mla::kWoOut) return MLA_ERR_BAD_DIM;
  if (!aligned16(x) || !aligned16(wo) || !stride8(x_sb) || (reinterpret_cast<uintptr_t>(out) & 1u) != 0)
    return MLA_ERR_ALIGNMENT;
  for (int32_t b0 = 0; b0 < B; b0 += 64) {
    mla::OutProjArgs a;
    a.x = static_cast<const uint16_t*>(x) + (int64_t)b0 * x_sb;
    a.wo = static_cast<const uint16_t*>(wo);
    a.out = static_cast<uint16_t*>(out) + (int64_t)b0 * out_sb;
    a.x_sb = x_sb;
    a.out_sb = out_sb;
    a.B = B - b0 < 64 ? B - b0 : 64;
    const int st = hip_status(mla::launch_output_proj(a, stream));
    if (st != MLA_OK) return st;
  }
  return MLA_OK;
}

int mla_combine_value_up(const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                         const void* wkv_b, void* out, int64_t out_sb, int64_t out_sh, float* lse,
                         uint32_t* status_dev, void* stream) {
  if (B < 1 || B > 65536 || num_splits < 2 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_BAD_DIM;
  if (!workspace || !wkv_b || !out) return MLA_ERR_NULL_POINTER;
  if (!aligned16(workspace) || !aligned16(wkv_b) || !aligned16(out) || !stride8(out_sb) || !stride8(out_sh))
    return MLA_ERR_ALIGNMENT;
  if (ws_bytes < mla_workspace_bytes(B, num_splits)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  const size_t units = (size_t)num_splits * (size_t)B * MLA_HEADS;
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
  a.lse = lse;
  a.status = status_dev;
  return hip_status(mla::launch_value_up(a, stream));
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
