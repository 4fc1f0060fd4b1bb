// The body of K1 (the decoupled RoPE channel and the paged cache write) as a
// per-block device function, shared by its own launch (rope.hip) and by the
// launch that also absorbs the query (gemm.hip).
#pragma once

#include "common.hpp"

namespace mla {

template <typename T> __device__ __forceinline__ double ld(const T* p, int64_t i);
template <> __device__ __forceinline__ double ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ double ld<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename T> __device__ __forceinline__ void st(T* p, int64_t i, double v);
template <> __device__ __forceinline__ void st<float>(float* p, int64_t i, double v) { p[i] = static_cast<float>(v); }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, int64_t i, double v) {
  p[i] = f32_to_bf16(static_cast<float>(v));
}

template <typename T, typename TO>
__device__ __forceinline__ void rotate_pairs(const RopeParams& p, const T* src, TO* dst, int pos, int lane,
                                             double scale) {
  const int half = p.d_rope / 2;
  for (int j = lane; j < half; j += 64) {
    double s, c;
    sincos(static_cast<double>(pos) * p.theta[j], &s, &c);
    const double x0 = ld(src, 2 * j), x1 = ld(src, 2 * j + 1);
    st(dst, 2 * j, (x0 * c - x1 * s) * scale);
    st(dst, 2 * j + 1, (x0 * s + x1 * c) * scale);
  }
}

// Blocks [0, rope_query_blocks): one query each.  Blocks after that: four
// cache rows each.  Queries without 16-byte vectors (q_vec == 0) take one wave
// per row.  `block` is the block's index in that numbering; 256 threads.
template <typename T, typename TQ>
__device__ __forceinline__ void rope_block(const RopeParams& p, int64_t block) {
  const int lane = threadIdx.x % 64;
  const int64_t width = p.d_latent + p.d_rope;
  const int half = p.d_rope / 2;
  const bool vec = p.q_vec != 0;
  const int64_t q_blocks = vec ? p.n_q : (p.n_q * p.n_heads + 3) / 4;
  if (block < q_blocks) {
    if (!vec) {
      const int64_t row = block * 4 + threadIdx.x / 64;
      if (row >= p.n_q * p.n_heads) return;
      const T* src = static_cast<const T*>(p.q_rope) + row * p.d_rope;
      TQ* dst = static_cast<TQ*>(p.q_lat) + row * width + p.d_latent;
      rotate_pairs<T, TQ>(p, src, dst, p.q_pos[row / p.n_heads], lane, p.q_scale);
      return;
    }
    __shared__ double cs[64], sn[64];
    const int64_t n = block;
    const int pos = p.q_pos[n];
    if (threadIdx.x < half) sincos(static_cast<double>(pos) * p.theta[threadIdx.x], &sn[threadIdx.x], &cs[threadIdx.x]);
    __syncthreads();
    // 8 consecutive elements (4 pairs) of one head per step
    const int per_head = p.d_rope / 8;
    const int pieces = p.n_heads * per_head;
    for (int k = threadIdx.x; k < pieces; k += 256) {
      const int h = k / per_head, e0 = (k % per_head) * 8;
      const int64_t row = n * p.n_heads + h;
      const T* src = static_cast<const T*>(p.q_rope) + row * p.d_rope + e0;
      TQ* dst = static_cast<TQ*>(p.q_lat) + row * width + p.d_latent + e0;
      T x[8];
      __builtin_memcpy(x, __builtin_assume_aligned(src, 16), sizeof(x));
      TQ y[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = e0 / 2 + i;
        const double x0 = ld(x, 2 * i), x1 = ld(x, 2 * i + 1);
        const double c = cs[j], sj = sn[j];
        st(y, 2 * i, (x0 * c - x1 * sj) * p.q_scale);
        st(y, 2 * i + 1, (x0 * sj + x1 * c) * p.q_scale);
      }
      __builtin_memcpy(__builtin_assume_aligned(dst, 16), y, sizeof(y));
    }
    return;
  }
  const int64_t m = (block - q_blocks) * 4 + threadIdx.x / 64;
  if (m >= p.n_kv) return;
  const int b = p.kv_seq[m];
  const int pos = p.kv_pos[m];
  if (b < 0 || b >= p.num_seqs || pos < 0) return;
  const int lp = pos / kPage;
  if (lp >= p.max_pages) return;
  const int page = p.block_table[static_cast<int64_t>(b) * p.max_pages + lp];
  if (page < 0 || page >= p.num_pages) return;
  T* dst = static_cast<T*>(p.cache) + (static_cast<int64_t>(page) * kPage + pos % kPage) * width;
  const T* lat = static_cast<const T*>(p.kv_latent) + m * p.d_latent;
  for (int c = lane; c < p.d_latent; c += 64) dst[c] = lat[c];
  rotate_pairs<T, T>(p, static_cast<const T*>(p.k_rope) + m * p.d_rope, dst + p.d_latent, pos, lane, 1.0);
}

inline int64_t rope_blocks(const RopeParams& p) {
  const int64_t q_blocks = p.q_vec ? p.n_q : (p.n_q * p.n_heads + 3) / 4;
  return q_blocks + (p.n_kv + 3) / 4;
}

}  // namespace mla
