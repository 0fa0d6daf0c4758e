// Internal interface between the C-ABI entry points (mla_api.cpp) and the
// HIP kernels (mla_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kHeads = 128;
constexpr int kNope = 128;
constexpr int kRope = 64;
constexpr int kLatent = 512;
constexpr int kValue = 128;
constexpr int kRowsPerHead = kNope + kValue;  // 256 rows of wkv_b per head
constexpr int kIdxCap = 2048;                  // index slots staged per split

// Block-scaled fp8 weight (read instead of wkv_b when w_fp8 != NULL): E4M3FN
// codes [32768][512] and fp32 scales [256][4], one per 128 x 128 block.
struct Fp8Weight {
  const uint8_t* w_fp8;
  const float* w_scale;
  uint16_t* w_formed;       // test hook: the bf16 weights as formed in registers (may be NULL)
};

struct AbsorbArgs {
  const uint16_t* q_nope;
  int64_t q_sb, q_sh;
  const uint16_t* wkv_b;
  uint16_t* q_abs;
  int32_t B;
  int32_t H;                // heads (128, or a head-sharded share: 16, 32, 64)
  Fp8Weight fp8;
};

struct DecodeArgs {
  const uint16_t* q_abs;
  const uint16_t* q_pe;
  int64_t q_pe_sb, q_pe_sh;
  const uint16_t* kv;
  int64_t kv_sb, kv_st;
  const uint16_t* pe;
  int64_t pe_sb, pe_st;
  const int32_t* seq_lens;
  const int32_t* indices;   // NULL: dense
  int32_t max_len;
  int32_t k_max;
  int32_t chunk;            // index slots per split (multiple of 32)
  int32_t B;                // query rows (sequences in decode, B * T tokens in prefill)
  int32_t H;                // heads (128, or a head-sharded share: 16, 32, 64)
  int32_t S;                // splits
  int32_t causal;           // 0: decode (row b = sequence b, length seq_lens[b]);
                            // 1: prefill, row r = token r % T of prompt r / T
                            // (T = rows_per_seq), causal length r % T + 1, no seq_lens
  int32_t rows_per_seq;
  float scale;              // softmax scale
  float scale_log2;         // softmax scale * log2(e)
  uint16_t* part_o;         // [S][B][128][512] bf16, unnormalised sum per split (S > 1)
  float* part_ml;           // [S][B][128][2]   (max, sum) per split      (S > 1)
  uint16_t* o_latent;       // [B][128][512]    when S == 1
  float* lse;               // [B][128]         when S == 1 (may be NULL)
  uint32_t flags;
  uint32_t* bitmap;
  int64_t bitmap_words;
  float* scores;            // [B][128][k_max]
  uint32_t* status;
};

struct CombineArgs {
  const uint16_t* part_o;
  const float* part_ml;
  int32_t B, S;
  int32_t H;
  uint16_t* o_latent;
  float* lse;
  uint32_t* status;
};

struct ValueUpArgs {
  const uint16_t* o_latent;  // [B][128][512]; NULL when the split partials are combined here
  const uint16_t* wkv_b;
  uint16_t* out;
  int64_t out_sb, out_sh;
  int32_t B;
  int32_t H;
  // Fused combine (o_latent == NULL): partials of mla_sparse_decode.
  const uint16_t* part_o;
  const float* part_ml;
  int32_t S;
  float* lse;
  uint32_t* status;
  Fp8Weight fp8;
};

struct DequantArgs {
  const uint8_t* w;
  const float* scales;
  uint16_t* out;
};

// Output projection: out[b][o] = sum_i x[b][i] wo[o][i], at most 64 rows.
constexpr int kWoIn = kHeads * kValue;  // 16384: the head outputs flattened
constexpr int kWoOut = 7168;            // model width
struct OutProjArgs {
  const uint16_t* x;    // [B][x_sb], the first kWoIn values of each row used
  const uint16_t* wo;   // [kWoOut][kWoIn]
  uint16_t* out;        // [B][out_sb], the first kWoOut values of each row written
  int64_t x_sb, out_sb;
  int32_t B;            // 1 .. 64
  bool packed;          // wo in the layout written by launch_output_proj_pack
  float* part;          // launch_output_proj_split: [kOpSplit][B][kWoOut] fp32 partial sums
};
// K-split output projection: workgroup = 4 x 28 outputs over a quarter of
// the inputs, the quarters' fp32 partial sums added by a second launch.
constexpr int kOpSplit = 4;

// Each returns a hipError_t value (0 on success).
int launch_absorb(const AbsorbArgs& a, void* stream);
int launch_decode(const DecodeArgs& a, void* stream);
int launch_combine(const CombineArgs& a, void* stream);
int launch_value_up(const ValueUpArgs& a, void* stream);  // fused combine when o_latent == NULL
// From this many merged rows on (o_latent given) the value-up streams tiles
// through workgroups that form W_UV,h once.
constexpr int kValueUpStreamMinRows = 512;
int launch_dequant(const DequantArgs& a, void* stream);
int launch_output_proj(const OutProjArgs& a, void* stream);
int launch_output_proj_pack(const uint16_t* wo, uint16_t* packed, void* stream);
int launch_output_proj_split(const OutProjArgs& a, void* stream);
int device_cu_count(int* cus);

// Static device scratch of mla_sparse_decode_noalloc: kScratchBytes per GPU.
constexpr size_t kScratchBytes = (size_t)40 << 20;
// The current device's scratch address (looked up once per device).
// Returns a hipError_t value (0 on success).
int scratch_buffer(void** ptr);

}  // namespace mla
