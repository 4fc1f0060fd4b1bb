// K2 (query absorption) and K6 (output absorption): per-head batched GEMMs.
//
// "AI decoupled RoPE MLA" (operatorworld.com), recap section: the two
// up-projections move to the two sides of attention -- W^UK^T onto the query
// (q~ = W^UK^T q, computed ahead of and independent of the cache) and W^UV
// after the weighted sum (Attn = W^UV sum_t alpha_t c_t).
//
// bf16 path: v_mfma_f32_16x16x32_bf16 with float32 accumulation.  Both GEMMs
// compute the transposed product (rows = output features, columns = tokens)
// so that each lane stores four consecutive output features of one token.
//  * absorb:   q~^T[j, n] = sum_i W_UK[h][i][j] q^C[n, h, i].  W_UK is stored
//    [d_h, d_c], so the MFMA A operand (8 consecutive i for one j) is a
//    column read: the W tile is staged in LDS and read with ds_read_tr16_b64.
//  * out_proj: o^T[v, n] = sum_j W_UV[h][v][j] obar[n, h, j].  Both operands
//    are already contiguous along j; obar is float32 and enters as a
//    two-term bf16 split; the float32 accumulator is stored as is (the
//    layer output is float32).
// float32 path: one thread per output element, float32 accumulation.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "decode_items.hpp"
#include "rope_block.hpp"

namespace mla {

namespace {

constexpr int kAbsorbJTile = 128;  // output features per workgroup
constexpr int kAbsorbLdsStride = kAbsorbJTile + 16;  // padded row (elements): 288 B
constexpr int kAbsorbNChunk = 512;  // most tokens per workgroup (looped in 64s)

// Tokens per workgroup for a grid of `per_chunk` workgroups per token chunk:
// the smallest multiple of 64 (at least 64, at most max_chunk) that keeps
// the grid within about `target` workgroups.  Small batches get one chunk
// (one load of each weight tile); long ones enough chunks to fill the chip.
inline int64_t token_chunk(int64_t n, int64_t per_chunk, int64_t target, int64_t max_chunk) {
  int64_t c = (n * per_chunk + target - 1) / target;
  c = (c + 63) / 64 * 64;
  return std::max<int64_t>(64, std::min<int64_t>(c, max_chunk));
}
static_assert((128 * (kAbsorbJTile / 8)) % 256 == 0, "W tile pieces must split evenly over the threads");

__device__ __forceinline__ bf16x8 load8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// W_UK tile [d_head rows (i), 128 cols (j)] in LDS; each wave owns 32 j x 64 n.
// A 64-token chunk of q^C goes through LDS once per workgroup (rows padded to
// 288 bytes: conflict-free fragment reads) instead of once per wave.
// One workgroup (256 threads) of the absorption: feature tile jt, head h,
// token chunk nz.
template <int DH, typename TQ>
__device__ __forceinline__ void absorb_block(const GemmParams& p, int jt, int h, int nz) {
  __shared__ __attribute__((aligned(16))) bf16_t w_lds[DH * kAbsorbLdsStride];
  constexpr int QS = DH + 16;  // q^C row stride in LDS (elements)
  __shared__ __attribute__((aligned(16))) bf16_t q_lds[64 * QS];
  const int j0 = jt * kAbsorbJTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int H = p.n_heads;
  const int DC = p.d_latent;
  const int D = p.d_latent + p.d_rope;
  const bf16_t* w = static_cast<const bf16_t*>(p.w) + static_cast<int64_t>(h) * DH * DC;
  const bf16_t* q = static_cast<const bf16_t*>(p.a);
  TQ* out = static_cast<TQ*>(p.out);
  const int64_t n_begin = static_cast<int64_t>(nz) * p.n_chunk;
  const int64_t n_end = min(p.n, n_begin + p.n_chunk);
  const int q16 = lane >> 4, r16 = lane & 15;
  const int jw = wave * 32;  // this wave's j offset inside the tile
  // A chunk of q^C (64 tokens x DH): this thread's 16-byte pieces, loaded
  // together and then stored to LDS.
  constexpr int QPT = 64 * (DH / 8) / 256;  // pieces per thread
  static_assert(QPT * 256 == 64 * (DH / 8), "q chunk pieces must split evenly over the threads");
  bf16x8 qv[QPT];
  auto load_q = [&](int64_t nb0) {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int c = tid + k * 256;
      const int r = c / (DH / 8), cc = c % (DH / 8);
      const int64_t n = nb0 + r;
      qv[k] = n < n_end ? load8(q + (n * H + h) * DH + cc * 8) : bf16x8{};
    }
  };
  auto store_q = [&] {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int c = tid + k * 256;
      const int r = c / (DH / 8), cc = c % (DH / 8);
      *reinterpret_cast<bf16x8*>(&q_lds[r * QS + cc * 8]) = qv[k];
    }
  };
  // The first chunk's queries load together with the W tile: one memory round trip.
  load_q(n_begin);
  // stage W_UK[h][:, j0 : j0 + 128]: all of this thread's loads, then all its LDS stores
  constexpr int WPT = DH * (kAbsorbJTile / 8) / 256;  // 16-byte pieces per thread
  bf16x8 wv[WPT];
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int c = tid + k * 256;
    const int row = c / (kAbsorbJTile / 8), cc = c % (kAbsorbJTile / 8);
    wv[k] = load8(w + static_cast<int64_t>(row) * DC + j0 + cc * 8);
  }
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int c = tid + k * 256;
    const int row = c / (kAbsorbJTile / 8), cc = c % (kAbsorbJTile / 8);
    *reinterpret_cast<bf16x8*>(&w_lds[row * kAbsorbLdsStride + cc * 8]) = wv[k];
  }
  store_q();
  __syncthreads();
  for (int64_t nb0 = n_begin; nb0 < n_end; nb0 += 64) {
    if (nb0 != n_begin) {
      load_q(nb0);
      __syncthreads();  // every wave is done with the previous chunk
      store_q();
      __syncthreads();
    }
    // B fragments of the chunk: token nb*16 + r16, i = ks*32 + q16*8 .. +7
    bf16x8 bq[DH / 32][4];
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        bq[ks][nb] = *reinterpret_cast<const bf16x8*>(&q_lds[(nb * 16 + r16) * QS + ks * 32 + q16 * 8]);
    f32x4 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        // A = W^T[j, i]: group q16 takes rows i0 .. i0+7 of column block jcol
        const int i0 = ks * 32 + q16 * 8;
        const int jcol = jw + jb * 16 + 4 * (r16 & 3);
        const int rr = r16 >> 2;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(&w_lds[(i0 + rr) * kAbsorbLdsStride + jcol]));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(&w_lds[(i0 + 4 + rr) * kAbsorbLdsStride + jcol]));
        bf16x8 a;
        __builtin_memcpy(&a, &lo, 8);
        __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[jb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq[ks][nb], acc[jb][nb], 0, 0, 0);
      }
    }
    // D^T[j][n]: lane holds n = nb*16 + r16, j = jb*16 + 4*q16 + e
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t n = nb0 + nb * 16 + r16;
      if (n >= n_end) continue;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int j = j0 + jw + jb * 16 + 4 * q16;
        if constexpr (sizeof(TQ) == 4) {
          *reinterpret_cast<f32x4*>(out + (n * H + h) * D + j) = acc[jb][nb];
        } else {
          uint2 packed;
          packed.x = pack_bf16x2(acc[jb][nb][0], acc[jb][nb][1]);
          packed.y = pack_bf16x2(acc[jb][nb][2], acc[jb][nb][3]);
          *reinterpret_cast<uint2*>(out + (n * H + h) * D + j) = packed;
        }
      }
    }
  }
}

// Work index w of the absorption: feature tile fastest, then head, then token
// chunk.  Through xcd_local the four feature tiles of a head (which read the
// same q^C chunk) share an XCD, so that chunk comes from HBM once.
template <int DH, typename TQ>
__device__ __forceinline__ void absorb_work(const GemmParams& g, int64_t a, int64_t n_abs) {
  const int64_t w = xcd_local(a, n_abs);
  const int jt_n = g.d_latent / kAbsorbJTile;
  const int64_t hn = w / jt_n;
  absorb_block<DH, TQ>(g, static_cast<int>(w % jt_n), static_cast<int>(hn % g.n_heads),
                       static_cast<int>(hn / g.n_heads));
}

template <int DH, typename TQ>
__global__ void __launch_bounds__(256) absorb_bf16_kernel(GemmParams p) {
  absorb_work<DH, TQ>(p, blockIdx.x, gridDim.x);
}

// The query prologue in one launch: blocks [0, n_rope) run K1 (query rotation
// and cache rows), blocks [r_pad, r_pad + n_abs) absorb (r_pad = n_rope rounded
// up to 32, so the absorption's XCD grouping holds; blocks in between exit).
// The two write disjoint columns of q_lat and share nothing else, so their
// blocks run side by side; the rotation's blocks come first so that its
// float64 angle chains start at once and end under the absorption.
template <int DH, typename T, typename TQ>
__global__ void __launch_bounds__(256) rope_absorb_kernel(GemmParams g, RopeParams r, int64_t n_rope, int64_t r_pad,
                                                          int64_t n_abs) {
  const int64_t blk = blockIdx.x;
  if (blk < n_rope)
    rope_block<T, TQ>(r, blk);
  else if (blk >= r_pad)
    absorb_work<DH, TQ>(g, blk - r_pad, n_abs);
}

// o^T[v, n] = W_UV[h][v, :] . obar[n, h, :].  A workgroup takes one head, 64
// rows v and a group of tokens (n_chunk, sized by the launcher to fill the
// chip); each of its four waves keeps its 16 rows of W_UV[h] (all of d_c) in
// registers, loaded once, while its tokens go by in chunks of 64: a chunk of
// obar[:, h, :] is staged in LDS once and read by all four waves.  So W_UV is
// read once per token group and obar once from HBM (its second reader, the
// other 64-row half of d_v, runs on the same XCD and finds it in L2).
// TO is obar's element type; a float32 obar is staged as a two-term bf16
// split hi + lo and takes two MFMAs per step, so it enters at ~16
// significant bits.
constexpr int kOutRows = 64;     // v rows per workgroup
constexpr int kOutChunk = 64;    // tokens per chunk
template <typename TO, int KMAX>
__global__ void __launch_bounds__(256) out_proj_bf16_kernel(GemmParams p) {
  constexpr int NTERM = sizeof(TO) == 4 ? 2 : 1;
  constexpr int LSTRIDE = KMAX + 8;  // bf16 elements per staged row (padding against bank conflicts)
  __shared__ __attribute__((aligned(16))) bf16_t ob_lds[NTERM][kOutChunk * LSTRIDE];
  // work index w = head * (d_v / 64) + row block; through xcd_local the row
  // blocks of a head (which read the same obar rows) share an XCD, so obar
  // comes from HBM once
  const int H = p.n_heads, DC = p.d_latent, DV = p.d_v;
  const int64_t wk = xcd_local(blockIdx.x, gridDim.x);
  const int64_t hw = wk / (DV / kOutRows);  // token group * H + head
  const int h = static_cast<int>(hw % H);
  const int64_t t_begin = (hw / H) * p.n_chunk, t_end = min(p.n, t_begin + p.n_chunk);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int v0 = static_cast<int>(wk % (DV / kOutRows)) * kOutRows + wave * 16;
  const int q16 = lane >> 4, r16 = lane & 15;
  const int ks_n = DC / 32;
  const bf16_t* w = static_cast<const bf16_t*>(p.w) + (static_cast<int64_t>(h) * DV + v0 + r16) * DC + q16 * 8;
  const TO* ob = static_cast<const TO*>(p.a);
  float* out = static_cast<float*>(p.out);
  // A fragments: W_UV[h][v0 + r16][k*32 + q16*8 .. +7] for every k step
  bf16x8 wa[KMAX / 32];
#pragma unroll
  for (int k = 0; k < KMAX / 32; ++k)
    if (k < ks_n) wa[k] = load8(w + k * 32);
  for (int64_t c0 = t_begin; c0 < t_end; c0 += kOutChunk) {
    const int rows = static_cast<int>(min<int64_t>(kOutChunk, t_end - c0));
    // stage obar[c0 .. c0 + rows, h, :] (zeros past the end)
    __syncthreads();
    // all of this thread's loads first, then its LDS stores: one round trip
    const int pieces = DC / 8;  // 8-element pieces per row
    constexpr int PPT = kOutChunk * (KMAX / 8) / 256;  // pieces per thread at the largest d_c
    bf16x8 v[NTERM][PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int c = tid + k * 256;
      const int r = c / pieces, pc = c % pieces;
      const bool ok = c < kOutChunk * pieces && r < rows;
      const TO* src = ob + ((c0 + r) * H + h) * DC + pc * 8;
      if constexpr (NTERM == 1) {
        v[0][k] = ok ? load8(src) : bf16x8{};
      } else {
        f32x4 x0 = ok ? *reinterpret_cast<const f32x4*>(src) : f32x4{};
        f32x4 x1 = ok ? *reinterpret_cast<const f32x4*>(src + 4) : f32x4{};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = e < 4 ? x0[e] : x1[e - 4];
          const __bf16 hi = static_cast<__bf16>(x);
          v[0][k][e] = hi;
          v[NTERM - 1][k][e] = static_cast<__bf16>(x - static_cast<float>(hi));
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NTERM; ++t)
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int c = tid + k * 256;
        const int r = c / pieces, pc = c % pieces;
        if (c < kOutChunk * pieces) *reinterpret_cast<bf16x8*>(&ob_lds[t][r * LSTRIDE + pc * 8]) = v[t][k];
      }
    __syncthreads();
    f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KMAX / 32; ++k) {
      if (k < ks_n) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int t = 0; t < NTERM; ++t) {
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&ob_lds[t][(nb * 16 + r16) * LSTRIDE + k * 32 + q16 * 8]);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[k], bv, acc[nb], 0, 0, 0);
          }
      }
    }
    // D^T[v][n]: lane holds n = nb*16 + r16, v = v0 + 4*q16 + e
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int r = nb * 16 + r16;
      if (r < rows) *reinterpret_cast<f32x4*>(out + ((c0 + r) * H + h) * DV + v0 + 4 * q16) = acc[nb];
    }
  }
}

// K4 + K6 in one launch: the split merge of a decode call and the output
// absorption, o[b, h, :] = W_UV[h] obar[b, h, :], where obar[b, h, :] is the
// lse-weighted sum of the sequence's split partials (every work item of the
// call left one, a sequence of one item included).  A workgroup of 8 waves
// takes one head and 16 sequences:
//  * 32 threads per sequence merge its row, DC/32 columns each, split by
//    split in index order with the arithmetic of merge_kernel, so obar has
//    the bits mla_decode's merge gives it;
//  * the merged rows go to LDS as a two-term bf16 split (as out_proj stages
//    a float32 obar) and never to HBM;
//  * wave w multiplies rows 16w .. 16w+15 of W_UV[h] with them: the MFMA
//    sequence of out_proj_bf16_kernel, so o has the bits mla_out_proj gives
//    it.  Two workgroups fit a CU (128 registers a lane).
// Work index = head * (sequence groups) + group; through xcd_local the groups
// of a head share an XCD and so W_UV[h] comes from HBM once per run of four.
constexpr int kMpSeqs = 16;   // sequences per workgroup
constexpr int kMpRows = 128;  // d_v rows per workgroup: 8 waves x 16
template <int DC, bool HALF>
__global__ void __launch_bounds__(512, 4) merge_proj_kernel(GemmParams g, AttnParams a) {
  constexpr int LSTRIDE = DC + 8;  // bf16 elements per staged row
  constexpr int CPT = DC / 32;     // merged columns per thread
  constexpr int U = 4;             // splits per load round
  __shared__ __attribute__((aligned(16))) bf16_t ob_lds[2][kMpSeqs * LSTRIDE];
  const int H = g.n_heads, DV = g.d_v;
  const int64_t n_grp = (g.n + kMpSeqs - 1) / kMpSeqs;
  const int64_t wk = xcd_local(blockIdx.x, gridDim.x);
  const int h = static_cast<int>(wk / n_grp);
  const int64_t s_begin = (wk % n_grp) * kMpSeqs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q16 = lane >> 4, r16 = lane & 15;
  // this thread's sequence and columns; its split count and first slot
  const int sq = tid >> 5, l32 = tid & 31;
  const int col = l32 * CPT;
  const int64_t b = s_begin + sq;
  const int64_t s_end = min(g.n, s_begin + kMpSeqs);
  // W_UV[h] rows v0 + r16, all of d_c, as MFMA A fragments.  With float16
  // partials the first half goes out first, under the loads of the lengths
  // and the partials (its addresses need neither); the rest after the merge,
  // when the partials' registers are free (all of it at once would not fit
  // two workgroups a CU).  Float32 partials take twice the registers, so
  // there all of it waits for the merge.
  constexpr int KW0 = HALF ? DC / 64 : 0;
  const int v0 = wave * 16;
  const bf16_t* w = static_cast<const bf16_t*>(g.w) + (static_cast<int64_t>(h) * DV + v0 + r16) * DC + q16 * 8;
  bf16x8 wa[DC / 32];
#pragma unroll
  for (int k = 0; k < KW0; ++k) wa[k] = load8(w + k * 32);
  const int L = a.split_pages;
  int ns = 0;
  int64_t base = 0;
  for (int64_t b0 = 0; b0 < s_end; b0 += 64) {
    const int64_t bb = b0 + lane;
    int t = bb < g.n ? a.seq_lens[bb] : 0;
    t = t < 0 ? 0 : t;
    const int pages = (t + kPage - 1) / kPage;
    const int nsl = pages / L + ((pages % L) != 0 ? 1 : 0);
    const int incl = wave_incl_scan(nsl);
    const int64_t rel = b - b0;
    const int src = static_cast<int>(rel < 0 ? 0 : rel > 63 ? 63 : rel);
    const int ns_src = __shfl(nsl, src, 64), incl_src = __shfl(incl, src, 64), total = __shfl(incl, 63, 64);
    if (rel >= 64) {
      base += total;
    } else if (rel >= 0) {
      ns = ns_src;
      base += incl_src - ns_src;
    }
  }
  if (b >= g.n || base + ns > a.n_items) ns = 0;
  const int64_t row0 = base * H + h;  // split s at partial row row0 + s * H
  const float* lse_s = a.ws_lse + row0;
  const float* part = a.ws_o + row0 * DC + col;
  const _Float16* hpart = reinterpret_cast<const _Float16*>(a.ws_o) + row0 * DC + col;
  const int32_t* pexp = HALF ? a.ws_exp + row0 * (DC / 128) + col / 128 : nullptr;
  // a round's partials stay in their stored type until used, as 32-bit words
  // (float16 ones two to a register: half the registers of their values)
  using PT = typename std::conditional<HALF, _Float16, float>::type;
  constexpr int VW = CPT * static_cast<int>(sizeof(PT)) / 4;
  uint32_t v[U][VW];
  int vex[U];
  float wl[U];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < ns) {
        const int64_t so = static_cast<int64_t>(s0 + u) * H;
        if constexpr (HALF) {
          __builtin_memcpy(v[u], hpart + so * DC, VW * 4);
          vex[u] = pexp[so * (DC / 128)];
        } else {
          __builtin_memcpy(v[u], part + so * DC, VW * 4);
        }
        wl[u] = lse_s[so];
      } else {
#pragma unroll
        for (int i = 0; i < VW; ++i) v[u][i] = 0;
        vex[u] = 0;
        wl[u] = -INFINITY;
      }
    }
  };
  load_round(0);
  // max of the splits' lse: the sequence's 32 threads take splits side by side
  float m = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 32)
    if (s0 + l32 < ns) m = fmaxf(m, lse_s[static_cast<int64_t>(s0 + l32) * H]);
#pragma unroll
  for (int k = 1; k < 32; k <<= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
  float acc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int s0 = 0; s0 < ns; s0 += U) {
      if (s0 > 0) load_round(s0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wu = __expf(wl[u] - m);
        wsum += wu;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          float x;
          if constexpr (HALF)
            x = ldexpf(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v[u][i / 2] >> (16 * (i % 2))))),
                       vex[u]);
          else
            x = __builtin_bit_cast(float, v[u][i]);
          acc[i] = fmaf(wu, x, acc[i]);
        }
      }
    }
  }
#pragma unroll
  for (int k = KW0; k < DC / 32; ++k) wa[k] = load8(w + k * 32);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (a.lse != nullptr && l32 == 0 && b < g.n) a.lse[b * H + h] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
  // stage obar (zeros for rows past the batch) as hi + lo.  No contraction
  // here: x must be rounded to float32 before lo = x - hi, as when out_proj
  // reads a stored obar (an fma would take lo from the unrounded product)
#pragma unroll
  for (int c8 = 0; c8 < CPT / 8; ++c8) {
#pragma clang fp contract(off)
    bf16x8 hi8, lo8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = acc[c8 * 8 + e] * inv;
      const __bf16 hi = static_cast<__bf16>(x);
      hi8[e] = hi;
      lo8[e] = static_cast<__bf16>(x - static_cast<float>(hi));
    }
    *reinterpret_cast<bf16x8*>(&ob_lds[0][sq * LSTRIDE + col + c8 * 8]) = hi8;
    *reinterpret_cast<bf16x8*>(&ob_lds[1][sq * LSTRIDE + col + c8 * 8]) = lo8;
  }
  __syncthreads();
  f32x4 acc_o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < DC / 32; ++k)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&ob_lds[t][r16 * LSTRIDE + k * 32 + q16 * 8]);
      acc_o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[k], bv, acc_o, 0, 0, 0);
    }
  // D^T[v][n]: lane holds sequence s_begin + r16, rows v0 + 4 q16 .. + 3
  if (s_begin + r16 < s_end)
    *reinterpret_cast<f32x4*>(static_cast<float*>(g.out) + ((s_begin + r16) * H + h) * DV + v0 + 4 * q16) = acc_o;
}

__global__ void __launch_bounds__(256) absorb_f32_kernel(GemmParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int DC = p.d_latent, DH = p.d_head, H = p.n_heads;
  if (idx >= p.n * H * DC) return;
  const int j = idx % DC;
  const int64_t nh = idx / DC;
  const int h = nh % H;
  const float* q = static_cast<const float*>(p.a) + nh * DH;
  const float* w = static_cast<const float*>(p.w) + static_cast<int64_t>(h) * DH * DC + j;
  float acc = 0.f;
  for (int i = 0; i < DH; ++i) acc = fmaf(q[i], w[static_cast<int64_t>(i) * DC], acc);
  static_cast<float*>(p.out)[nh * (DC + p.d_rope) + j] = acc;
}

// One wave per output o[n, h, v]: the lanes walk the W_UV row and the obar row
// side by side (coalesced), then sum across the wave in a fixed order.
__global__ void __launch_bounds__(256) out_proj_f32_kernel(GemmParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int DC = p.d_latent, DV = p.d_v, H = p.n_heads;
  if (idx >= p.n * H * DV) return;
  const int v = idx % DV;
  const int64_t nh = idx / DV;
  const int h = nh % H;
  const float* ob = static_cast<const float*>(p.a) + nh * DC;
  const float* w = static_cast<const float*>(p.w) + (static_cast<int64_t>(h) * DV + v) * DC;
  float acc = 0.f;
  for (int j = lane; j < DC; j += 64) acc = fmaf(w[j], ob[j], acc);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) acc += __shfl_xor(acc, k, 64);
  if (lane == 0) static_cast<float*>(p.out)[idx] = acc;
}

}  // namespace

namespace {
// workgroups of the bf16 absorption, with p.n_chunk set
int64_t absorb_grid(GemmParams& p) {
  const int64_t per_chunk = static_cast<int64_t>(p.d_latent / kAbsorbJTile) * p.n_heads;
  p.n_chunk = token_chunk(p.n, per_chunk, 1024, kAbsorbNChunk);
  return per_chunk * ((p.n + p.n_chunk - 1) / p.n_chunk);
}
}  // namespace

hipError_t launch_absorb(const GemmParams& p_in, hipStream_t s) {
  GemmParams p = p_in;
  if (p.n == 0) return hipSuccess;
  if (p.dtype == 0) {
    const int64_t total = p.n * p.n_heads * p.d_latent;
    hipLaunchKernelGGL(absorb_f32_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, p);
  } else {
    const dim3 grid(static_cast<unsigned>(absorb_grid(p)));
    if (p.work_dtype == 0)
      hipLaunchKernelGGL((absorb_bf16_kernel<128, float>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((absorb_bf16_kernel<128, bf16_t>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_rope_absorb(const GemmParams& g_in, const RopeParams& r, hipStream_t s) {
  // the fused launch covers the bf16 absorption; other types take the two launches
  if (g_in.dtype == 0 || g_in.n == 0) {
    hipError_t e = launch_rope(r, s);
    if (e != hipSuccess) return e;
    return launch_absorb(g_in, s);
  }
  GemmParams g = g_in;
  const int64_t n_abs = absorb_grid(g);
  const int64_t n_rope = rope_blocks(r);
  const int64_t r_pad = (n_rope + 31) / 32 * 32;
  const dim3 grid(static_cast<unsigned>(r_pad + n_abs));
  if (g.work_dtype == 0)
    hipLaunchKernelGGL((rope_absorb_kernel<128, bf16_t, float>), grid, dim3(256), 0, s, g, r, n_rope, r_pad, n_abs);
  else
    hipLaunchKernelGGL((rope_absorb_kernel<128, bf16_t, bf16_t>), grid, dim3(256), 0, s, g, r, n_rope, r_pad,
                       n_abs);
  return hipGetLastError();
}

hipError_t launch_merge_proj(const GemmParams& g, const AttnParams& a, hipStream_t s) {
  if (g.n == 0) return hipSuccess;
  if (g.d_v != kMpRows) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(g.n_heads * ((g.n + kMpSeqs - 1) / kMpSeqs)));
  if (g.d_latent == 512 && a.half_partials)
    hipLaunchKernelGGL((merge_proj_kernel<512, true>), grid, dim3(512), 0, s, g, a);
  else if (g.d_latent == 512)
    hipLaunchKernelGGL((merge_proj_kernel<512, false>), grid, dim3(512), 0, s, g, a);
  else if (g.d_latent == 256 && !a.half_partials)
    hipLaunchKernelGGL((merge_proj_kernel<256, false>), grid, dim3(512), 0, s, g, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_out_proj(const GemmParams& p_in, hipStream_t s) {
  GemmParams p = p_in;
  if (p.n == 0) return hipSuccess;
  if (p.dtype == 0) {
    const int64_t total = p.n * p.n_heads * p.d_v;
    if ((total + 3) / 4 > 0x7fffffff) return hipErrorInvalidValue;  // one wave per output: grid limit
    hipLaunchKernelGGL(out_proj_f32_kernel, dim3(static_cast<unsigned>((total + 3) / 4)), dim3(256), 0, s, p);
  } else {
    // token groups: enough workgroups to fill the chip (each loads its head's W_UV rows once)
    const int64_t per_group = static_cast<int64_t>(p.d_v / kOutRows) * p.n_heads;
    p.n_chunk = token_chunk(p.n, per_group, 512, (p.n + 63) / 64 * 64);
    const dim3 grid(static_cast<unsigned>(per_group * ((p.n + p.n_chunk - 1) / p.n_chunk)));
    if (p.d_latent <= 256)
      hipLaunchKernelGGL((out_proj_bf16_kernel<float, 256>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((out_proj_bf16_kernel<float, 512>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mla
