// float32 absorbed attention over the paged latent cache (decode and causal
// prefill), on the vector ALUs.  Same equations as the bf16 MFMA kernel
// ("AI decoupled RoPE MLA", decoupled-RoPE score; one scale on the summed
// score), kept in float32 end to end for the float32 workloads, where a
// bf16 rounding of the probabilities would exceed a 1e-4 budget.
//
// One workgroup (256 lanes) per row (query, head).  Keys are taken 256 at a
// time: lane k scores key k (a dot product of the 576- or 288-wide query with
// the cache row), the block forms the running max / sum, and then each lane
// accumulates its own latent columns over the 256 keys.  No split over the
// cache: this path is for small and latency-bound shapes.
#include "common.hpp"

namespace mla {

namespace {

constexpr int kF32Threads = 256;
constexpr int kF32MaxD = 1152;    // d_latent + d_rope upper bound
constexpr int kF32MaxPerLane = 4;  // d_latent <= 1024

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float o = __shfl_xor(v, m, 64);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kF32Threads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

template <bool PREFILL>
__global__ void __launch_bounds__(kF32Threads) attn_f32_kernel(AttnParams p) {
  __shared__ float q_s[kF32MaxD];
  __shared__ float p_s[kF32Threads];
  __shared__ const float* row_s[kF32Threads];
  __shared__ float red[kF32Threads / 64];
  const int tid = threadIdx.x;
  const int H = p.n_heads, DC = p.d_latent, D = p.d_latent + p.d_rope;
  const int64_t g = blockIdx.x;  // row = query * H + head
  const int64_t n = g / H;
  int b, key_end;
  if constexpr (PREFILL) {
    int lo = 0, hi = p.batch - 1;  // last b with cu_q[b] <= n
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (p.cu_q[mid] <= n) lo = mid; else hi = mid - 1;
    }
    b = lo;
    key_end = p.q_start[b] + static_cast<int>(n - p.cu_q[b]) + 1;
  } else {
    b = static_cast<int>(n);
    key_end = max(p.seq_lens[b], 0);
  }
  if (b >= p.num_seqs) return;
  const float* q = static_cast<const float*>(p.q_lat) + g * D;
  for (int i = tid; i < D; i += kF32Threads) q_s[i] = q[i];
  const float* cache = static_cast<const float*>(p.cache);
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const float scale = p.scale;
  float acc[kF32MaxPerLane];
#pragma unroll
  for (int i = 0; i < kF32MaxPerLane; ++i) acc[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();
  for (int k0 = 0; k0 < key_end; k0 += kF32Threads) {
    const int t = k0 + tid;
    float s = -INFINITY;
    const float* row = nullptr;
    if (t < key_end) {
      const int lp = t / kPage;
      int id = lp < p.max_pages ? bt[lp] : -1;
      id = (id < 0 || id >= p.num_pages) ? 0 : id;
      row = cache + (static_cast<int64_t>(id) * kPage + t % kPage) * D;
      float dot = 0.f;
      for (int i = 0; i < D; ++i) dot = fmaf(q_s[i], row[i], dot);
      s = dot * scale;
    }
    const float mx = block_reduce(s, red, true);
    const float m_new = fmaxf(m_run, mx);
    const float pk = t < key_end ? expf(s - m_new) : 0.f;
    const float corr = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
    const float psum = block_reduce(pk, red, false);
    l_run = l_run * corr + psum;
    m_run = m_new;
    p_s[tid] = pk;
    row_s[tid] = row;
    __syncthreads();
    const int nk = min(kF32Threads, key_end - k0);
#pragma unroll
    for (int i = 0; i < kF32MaxPerLane; ++i) {
      const int c = tid + i * kF32Threads;
      if (c >= DC) break;
      float a = acc[i] * corr;
      for (int k = 0; k < nk; ++k) a = fmaf(p_s[k], row_s[k][c], a);
      acc[i] = a;
    }
    __syncthreads();
  }
  float* out = static_cast<float*>(p.out_latent) + g * DC;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int i = 0; i < kF32MaxPerLane; ++i) {
    const int c = tid + i * kF32Threads;
    if (c < DC) out[c] = acc[i] * inv;
  }
  if (p.lse != nullptr && tid == 0) p.lse[g] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

}  // namespace

hipError_t launch_decode_f32(const AttnParams& p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.batch) * p.n_heads;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_f32_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(kF32Threads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const AttnParams& p, hipStream_t s) {
  const int64_t rows = p.n_blocks;  // total queries * heads
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_f32_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(kF32Threads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
