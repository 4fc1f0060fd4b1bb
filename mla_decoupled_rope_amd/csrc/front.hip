// The front of the layer: the projections from the hidden state h that feed
// the cache and the query.
//
// "AI decoupled RoPE MLA" (operatorworld.com), recap: the latent is the
// down-projection c_t = W^DKV h_t; decoupled-RoPE section: the small position
// channel k^R_t = W^KR h_t is the only part rotated, and the cache row is
// [c_t | R_t k^R_t].  "Detailed Illustration of the Problem" (notion.site),
// Step 1: the query goes through a compressed latent c^Q = W^DQ h and is
// projected up from it; Step 4: without a rotation in between, W^UK folds
// into the query weight (W^{Q'} = (W^UQ)^T W^UK), so the absorbed query
// q~ = W_UK^T W_UQ c^Q comes out of one projection.
//
// Every projection is Y = X W^T with X [M, K] tokens and W [N, K] (rows are
// output features), both K-contiguous, so both MFMA operands are plain
// 16-byte fragment reads:
//   gemm_nt_kernel   -- a 64-token x 128-feature tile per workgroup over one
//                       split of K, 4 waves of 32 x 64 on
//                       v_mfma_f32_32x32x16_bf16; X and W come through a ring
//                       of four 32-wide K slices filled by LDS DMA; float32
//                       partials [split][M][N].  Split-K keeps a decode-sized
//                       M (a few dozen tokens) streaming the weights from
//                       enough workgroups.
//   front_reduce     -- sums the splits in order (so results are bitwise
//                       repeatable) and writes the destination: bf16 rows
//                       (the query latent), the cache row with R_p k^R
//                       (float64 angles, like the RoPE kernel), or q^C to
//                       q_nope / q~ to q_lat and R_p q^R to q_lat's tail.
//   fold_kernel      -- W_fold,i = W_UK,i^T W_UQ,i, once per weight set
//                       (float32 sums, bf16 out).
#include "common.hpp"

namespace mla {

namespace {

constexpr int kGBM = 64;    // tokens per tile
constexpr int kGBN = 128;   // features per tile
constexpr int kGSl = 32;    // K per slice
constexpr int kGRing = 4;
constexpr int kBufWord3 = 0x00020000;  // raw buffer resource, 32-bit format (gfx9 family)

constexpr int vmcnt_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// LDS rows are 64 bytes (32 bf16); chunk ch of row r sits in slot ch ^ ((r >> 2) & 3),
// which puts the 16 rows of a fragment-read phase on distinct banks.
__device__ __forceinline__ int g_slot(int r, int ch) { return ch ^ ((r >> 2) & 3); }

__global__ void __launch_bounds__(256) gemm_nt_kernel(GemmNtParams p) {
  constexpr int RB = kGSl * 2;              // 64-byte rows
  constexpr int XB = kGBM * RB;             // 4 KiB of X a slice
  constexpr int SLB = XB + kGBN * RB;       // + 8 KiB of W
  __shared__ __attribute__((aligned(16))) char ring[kGRing * SLB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, kh = lane >> 5;
  const int n0 = blockIdx.x * kGBN, m0 = blockIdx.y * kGBM;
  const int split = blockIdx.z;
  const int k0 = split * p.k_split;
  const int ns = p.k_split / kGSl;          // slices

  // ---- DMA: instruction j of a slice: j < 4 -> X rows 16j .. +15; else W
  // rows 16(j-4) .. +15.  Wave w issues j = w, w + 4, w + 8.  Rows past M or
  // N repeat the last row (never stored).  A 16-row W group lies in one
  // weight segment (n1 is a multiple of 16).
  __amdgpu_buffer_rsrc_t rs[3];
  uint32_t off[3];
  int ldsoff[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int j = wave + 4 * k;
    const int slot = lane & 3;
    if (j < 4) {
      const int row = 16 * j + (lane >> 2);
      const int m = min(m0 + row, p.m - 1);
      rs[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.x), 0,
                                                static_cast<int>(static_cast<uint32_t>(
                                                    min(static_cast<int64_t>(p.m) * p.ldx * 2, int64_t{0xffffffff}))),
                                                kBufWord3);
      off[k] = static_cast<uint32_t>(static_cast<int64_t>(m) * p.ldx * 2 + g_slot(row, slot) * 16);
      ldsoff[k] = j * 1024;
    } else {
      const int row = 16 * (j - 4) + (lane >> 2);
      const int g0 = __builtin_amdgcn_readfirstlane(n0 + 16 * (j - 4));  // the group's first feature
      const int nf = min(n0 + row, p.n - 1);
      const bool seg1 = g0 < p.n1 || p.n1 == p.n;
      const bf16_t* base = seg1 ? p.w1 : p.w2;
      const int rows = seg1 ? p.n1 : p.n - p.n1;
      const int nr = seg1 ? nf : nf - p.n1;
      rs[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), 0,
                                                static_cast<int>(static_cast<uint32_t>(
                                                    min(static_cast<int64_t>(rows) * p.k * 2, int64_t{0xffffffff}))),
                                                kBufWord3);
      off[k] = static_cast<uint32_t>(static_cast<int64_t>(nr) * p.k * 2 + g_slot(row, slot) * 16);
      ldsoff[k] = XB + (j - 4) * 1024;
    }
  }
  auto buf = [&](int s) { return ring + (s % kGRing) * SLB; };
  auto issue = [&](int s) {
    lds_char_t* dst = reinterpret_cast<lds_char_t*>(reinterpret_cast<uintptr_t>(buf(s)));
    const int so = (k0 + s * kGSl) * 2;
#pragma unroll
    for (int k = 0; k < 3; ++k) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[k], dst + ldsoff[k], 16, off[k], so, 0, 0);
  };

  // ---- wave (wm, wn): tokens 32 wm .. +31, features 64 wn .. +63
  const int wm = wave & 1, wn = wave >> 1;
  int foff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) foff[ks] = r32 * RB + g_slot(r32, 2 * ks + kh) * 16;
  f32x16 acc[2] = {f32x16{}, f32x16{}};

  for (int s = 0; s < 3 && s < ns; ++s) issue(s);
  for (int s = 0; s < ns; ++s) {
    // slice s lands; this wave's three instructions of each newer slice may stay in flight
    const int newer = min(2, ns - 1 - s);
    if (newer == 2) __builtin_amdgcn_s_waitcnt(vmcnt_wait(6));
    else if (newer == 1) __builtin_amdgcn_s_waitcnt(vmcnt_wait(3));
    else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (s + 3 < ns) issue(s + 3);  // buffer (s+3) % 4 = (s-1) % 4: every wave is past it
    const char* sl = buf(s);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(sl + (32 * wm) * RB + foff[ks]);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const bf16x8 w = *reinterpret_cast<const bf16x8*>(sl + XB + (64 * wn + 32 * a) * RB + foff[ks]);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, b, acc[a], 0, 0, 0);
      }
    }
  }
  // ---- D[n][m]: lane (m = r32, half kh) holds n = 8g + 4kh + e at register 4g + e
  const int m = m0 + 32 * wm + r32;
  if (m >= p.m) return;
  float* out = p.part + (static_cast<int64_t>(split) * p.m + m) * p.n;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + 64 * wn + 32 * a + 8 * g + 4 * kh;
      if (n < p.n)
        *reinterpret_cast<f32x4*>(out + n) =
            f32x4{acc[a][4 * g], acc[a][4 * g + 1], acc[a][4 * g + 2], acc[a][4 * g + 3]};
    }
}

// One pair of features (2f, 2f + 1) of one token per thread.
template <int MODE>
__global__ void __launch_bounds__(256) front_reduce_kernel(FrontReduceParams p) {
  const int m = blockIdx.y;
  const int f = 2 * (blockIdx.x * 256 + threadIdx.x);
  if (f >= p.n) return;
  const int64_t stride = static_cast<int64_t>(p.m) * p.n;
  const float* src = p.part + static_cast<int64_t>(m) * p.n + f;
  double v0 = 0.0, v1 = 0.0;
  {
    // Splits are added in order; their loads go out eight at a time, so a
    // round costs one memory latency instead of eight.
    constexpr int U = 8;
    float s0 = 0.f, s1 = 0.f;
    int s = 0;
    for (; s + U <= p.splits; s += U) {
      float2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const float2*>(src + (s + u) * stride);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s0 += v[u].x;
        s1 += v[u].y;
      }
    }
    for (; s < p.splits; ++s) {
      const float2 v = *reinterpret_cast<const float2*>(src + s * stride);
      s0 += v.x;
      s1 += v.y;
    }
    v0 = s0;
    v1 = s1;
  }
  auto rot = [&](int pos, int j, double& x0, double& x1) {
    double sn, cs;
    sincos(static_cast<double>(pos) * p.theta[j], &sn, &cs);
    const double y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
    x0 = y0;
    x1 = y1;
  };
  auto put = [](bf16_t* dst, double a, double b) {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(static_cast<float>(a), static_cast<float>(b));
  };
  if constexpr (MODE == kFrontPlain) {
    put(p.y + static_cast<int64_t>(m) * p.ldy + f, v0, v1);
  } else if constexpr (MODE == kFrontKv) {
    // features [0, d_c): the latent; [d_c, d_c + d_r): k^R, rotated to the token's position
    const int seq = p.kv_seq[m], pos = p.kv_pos[m];
    if (seq < 0 || pos < 0) return;  // a row that is not written
    const int pg = pos / kPage;
    if (pg >= p.max_pages) return;
    const int page = p.block_table[static_cast<int64_t>(seq) * p.max_pages + pg];
    if (page < 0 || page >= p.num_pages) return;
    if (f >= p.d_latent) rot(pos, (f - p.d_latent) / 2, v0, v1);
    bf16_t* row = static_cast<bf16_t*>(p.cache) + (static_cast<int64_t>(page) * kPage + pos % kPage) *
                                                      (p.d_latent + p.d_rope);
    put(row + f, v0, v1);
  } else {
    // features [0, H * W0): q^C per head (W0 = d_head) or q~ per head (W0 = d_c);
    // [H * W0, H * (W0 + d_r)): q^R per head, rotated to the query's position
    constexpr bool folded = MODE == kFrontQFolded;
    const int w0 = folded ? p.d_latent : p.d_head;
    const int row_w = p.d_latent + p.d_rope;
    const int split = p.n_heads * w0;
    if (f < split) {
      const int h = f / w0, d = f % w0;
      if (folded)
        put(p.q_lat + (static_cast<int64_t>(m) * p.n_heads + h) * row_w + d, v0, v1);
      else
        put(p.q_nope + (static_cast<int64_t>(m) * p.n_heads + h) * p.d_head + d, v0, v1);
    } else {
      const int g = f - split, h = g / p.d_rope, d = g % p.d_rope;
      rot(p.q_pos[m], d / 2, v0, v1);
      v0 *= p.q_scale;  // the two-scale score's ratio, inside the one rounding
      v1 *= p.q_scale;
      put(p.q_lat + (static_cast<int64_t>(m) * p.n_heads + h) * row_w + p.d_latent + d, v0, v1);
    }
  }
}

// W_fold[h][c][j] = sum_i W_UK[h][i][c] W_UQ[h][i][j]: a 16 x 64 tile per workgroup,
// four outputs per thread.
__global__ void __launch_bounds__(256) fold_kernel(FoldParams p) {
  const int h = blockIdx.z;
  const int j = blockIdx.x * 64 + (threadIdx.x & 63);
  const int c0 = blockIdx.y * 16 + (threadIdx.x >> 6) * 4;
  if (j >= p.d_qlat) return;
  const bf16_t* uq = p.w_uq + static_cast<int64_t>(h) * p.d_head * p.d_qlat;
  const bf16_t* uk = p.w_uk + static_cast<int64_t>(h) * p.d_head * p.d_latent;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < p.d_head; ++i) {
    const float a = bf16_to_f32(uq[static_cast<int64_t>(i) * p.d_qlat + j]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (c0 + t < p.d_latent) acc[t] += bf16_to_f32(uk[static_cast<int64_t>(i) * p.d_latent + c0 + t]) * a;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (c0 + t < p.d_latent)
      p.w_fold[(static_cast<int64_t>(h) * p.d_latent + c0 + t) * p.d_qlat + j] = f32_to_bf16(acc[t]);
}

}  // namespace

hipError_t launch_gemm_nt(const GemmNtParams& p, int splits, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.n + kGBN - 1) / kGBN), static_cast<unsigned>((p.m + kGBM - 1) / kGBM),
                  static_cast<unsigned>(splits));
  hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_front_reduce(const FrontReduceParams& p, int mode, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.n / 2 + 255) / 256), static_cast<unsigned>(p.m));
  switch (mode) {
    case kFrontPlain: hipLaunchKernelGGL(front_reduce_kernel<kFrontPlain>, grid, dim3(256), 0, s, p); break;
    case kFrontKv: hipLaunchKernelGGL(front_reduce_kernel<kFrontKv>, grid, dim3(256), 0, s, p); break;
    case kFrontQ: hipLaunchKernelGGL(front_reduce_kernel<kFrontQ>, grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL(front_reduce_kernel<kFrontQFolded>, grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_fold(const FoldParams& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.d_qlat + 63) / 64), static_cast<unsigned>((p.d_latent + 15) / 16),
                  static_cast<unsigned>(p.n_heads));
  hipLaunchKernelGGL(fold_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
