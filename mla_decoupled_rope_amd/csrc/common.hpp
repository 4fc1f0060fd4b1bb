// Shared device helpers and the internal launcher interface of libmla.
// gfx950 (CDNA4) only: 64-wide waves, bf16 MFMA, LDS transpose reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPage = 64;  // tokens per cache page (one attention tile)
// Cache-policy operand of the buffer intrinsics (gfx950): the nt bit marks a
// load's lines for early eviction (data read once, as a decode streams the cache).
constexpr int kCpolNt = 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short bf16_t;  // storage type of a bf16 value
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round-to-nearest-even float -> bf16 by the hardware conversion
// (v_cvt_pk_bf16_f32; NaN stays NaN).  A software rounding with a NaN test
// costs a branch per value, which dominated the epilogues.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two floats to a packed bf16 pair (lo in bits 0-15), one conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Round-to-nearest-even float -> bf16 for values known to be finite.
__device__ __forceinline__ bf16_t f32_to_bf16_finite(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Reductions over lane pairs (l, l ^ 16) and (l, l ^ 32) with the gfx950
// permlane swaps: swapping a value with itself leaves each lane holding its own
// value in one result and its partner's in the other, so max/sum of the two
// results is the pair's max/sum.  Register-only, no LDS traffic.
__device__ __forceinline__ float pair16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------- params --

struct RopeParams {
  int n_heads, d_latent, d_rope, dtype, work_dtype;
  const void* q_rope; const int32_t* q_pos; int64_t n_q; void* q_lat;
  const void* kv_latent; const void* k_rope; const int32_t* kv_seq; const int32_t* kv_pos; int64_t n_kv;
  void* cache; int64_t num_pages; const int32_t* block_table; int32_t num_seqs; int32_t max_pages;
  int q_vec;  // query pairs in 16-byte vectors: d_rope % 8 == 0 and q_rope, q_lat 16-byte aligned
  double q_scale;    // rotated query times position_scale / softmax_scale (1 for one scale)
  double theta[64];  // theta_j, j < d_rope / 2 (float64, from the host)
};

struct GemmParams {
  int n_heads, d_head, d_v, d_latent, d_rope, dtype, work_dtype;
  const void* a; const void* w; void* out; int64_t n;
  int64_t n_chunk;  // tokens per workgroup (a multiple of 64; set by the launcher)
};

// Front of the layer: Y = X W^T in split-K partials, then a reduce that
// writes the projection's destination.
struct GemmNtParams {
  const bf16_t* x; int64_t ldx;           // [M, K] activations, row stride ldx elements
  const bf16_t* w1; const bf16_t* w2;     // weight rows [0, n1) from w1, [n1, n) from w2, each [rows, K]
  int m, n, n1, k, k_split;               // k_split: K elements per split (a multiple of 32)
  float* part;                            // [splits, M, N] float32
};

enum FrontMode { kFrontPlain = 0, kFrontKv = 1, kFrontQ = 2, kFrontQFolded = 3 };

struct FrontReduceParams {
  const float* part; int splits; int m, n;
  // plain: bf16 y [M, ldy]
  bf16_t* y; int64_t ldy;
  // shape
  int n_heads, d_head, d_latent, d_rope;
  // kv: the cache row [c | R_p k^R] of (kv_seq, kv_pos)
  void* cache; int64_t num_pages; const int32_t* block_table; int32_t max_pages;
  const int32_t* kv_seq; const int32_t* kv_pos;
  // q: q_nope [M, H, d_head], q_lat [M, H, d_latent + d_rope], positions
  bf16_t* q_nope; bf16_t* q_lat; const int32_t* q_pos;
  double q_scale;  // rotated query times position_scale / softmax_scale (1 for one scale)
  double theta[64];
};

struct FoldParams {
  const bf16_t* w_uq; const bf16_t* w_uk; bf16_t* w_fold;  // [H, d_h, d_q], [H, d_h, d_c] -> [H, d_c, d_q]
  int n_heads, d_head, d_latent, d_qlat;
};

hipError_t launch_gemm_nt(const GemmNtParams& p, int splits, hipStream_t s);
hipError_t launch_front_reduce(const FrontReduceParams& p, int mode, hipStream_t s);
hipError_t launch_fold(const FoldParams& p, hipStream_t s);

// Decode / prefill attention over the paged latent cache.
struct AttnParams {
  // shape
  int n_heads, d_latent, d_rope;
  int f32w;          // float32 working precision: float32 q_lat; q~ and P enter as two-term bf16
  float scale;       // softmax_scale
  float scale_log2;  // softmax_scale * log2(e)
  // inputs
  const void* q_lat; const void* cache; int64_t num_pages;
  const int32_t* block_table; int32_t num_seqs; int32_t max_pages;
  // decode
  const int32_t* seq_lens; int32_t batch; int32_t split_pages; int32_t n_full; int64_t n_items;
  int32_t n_head_chunks;
  // prefill
  const int32_t* cu_q; const int32_t* q_start; int64_t n_blocks;
  // outputs
  void* out_latent; float* lse;
  // split partials: normalised obar [slot, H, d_latent] / lse [slot, H].  With
  // half_partials the obar partials are float16 scaled by 2^-e per 128-column
  // quarter of a row (e = the quarter's largest magnitude's frexp exponent, so
  // every stored value is below 1 in magnitude), e in ws_exp [slot, H, d_latent / 128].
  float* ws_o; float* ws_lse;
  int half_partials; int32_t* ws_exp;
  // every decode work item writes a partial, a sequence of one item included
  // (for the fused merge and output absorption, which reads only partials)
  int all_partials;
};

// Materialised-form prefill: per-head keys and values up-projected from the
// latent cache into a workspace, then causal attention over them.
struct MhaParams {
  int n_heads, d_latent, d_rope;
  float scale_log2;  // softmax_scale * log2(e)
  const void* cache; int64_t num_pages;
  const int32_t* block_table; int32_t num_seqs; int32_t max_pages;
  const int32_t* cu_q; const int32_t* q_start; int32_t batch;
  const void* q_nope;  // [n_q, H, 128] bf16
  const void* q_lat;   // [n_q, H, d_latent + d_rope] bf16; only the rotated tail is read
  const void* w_uk; const void* w_uv;  // [H, 128, d_latent] bf16
  uint16_t* ws_k; uint16_t* ws_v;      // [H, n_keys, 128] float16
  int64_t n_keys;                      // sum over sequences of q_start + n_q
  int64_t n_key_tiles;                 // 256-key tiles of the up-projection (per head)
  int64_t n_q_blocks;                  // (sequence, 128-query block) pairs
  float* out; float* lse;              // [n_q, H, 128] float32 / [n_q, H]
};

// The debug-mode check of the paging data (MLA_DEBUG_VALIDATE=1): the
// lengths are seq_lens (decode) or q_start + (cu_q[b+1] - cu_q[b]) (prefill,
// when cu_q is set); kv_seq / kv_pos are the cache rows a call writes.
struct CheckParams {
  const int32_t* block_table; int32_t num_seqs; int32_t max_pages; int64_t num_pages;
  int32_t batch;
  const int32_t* seq_lens; const int32_t* cu_q; const int32_t* q_start;
  const int32_t* kv_seq; const int32_t* kv_pos; int64_t n_kv;
};
enum CheckKind { kCheckOk = 0, kCheckPage = 1, kCheckLength = 2, kCheckRow = 3 };
// Runs the check on stream s and waits for it: record = {kind, a, b, c,
// sum of the lengths, xor-hash of (length * 2654435761) ^ index}.
hipError_t run_check(const CheckParams& p, int32_t* record, hipStream_t s);

// Launchers (each returns hipGetLastError() after the launch).
hipError_t launch_rope(const RopeParams& p, hipStream_t s);
hipError_t launch_perhead_decode(const AttnParams& p, hipStream_t s);
hipError_t launch_perhead_cache_write(const RopeParams& p, hipStream_t s);
hipError_t launch_absorb(const GemmParams& p, hipStream_t s);
hipError_t launch_rope_absorb(const GemmParams& g, const RopeParams& r, hipStream_t s);
hipError_t launch_out_proj(const GemmParams& p, hipStream_t s);
hipError_t launch_decode_bf16(const AttnParams& p, hipStream_t s);
hipError_t launch_prefill_bf16(const AttnParams& p, hipStream_t s);
hipError_t launch_merge(const AttnParams& p, hipStream_t s);
hipError_t launch_merge_proj(const GemmParams& g, const AttnParams& a, hipStream_t s);
hipError_t launch_decode_f32(const AttnParams& p, hipStream_t s);
hipError_t launch_prefill_f32(const AttnParams& p, hipStream_t s);
hipError_t launch_mha_prefill(const MhaParams& p, hipStream_t s);

}  // namespace mla
