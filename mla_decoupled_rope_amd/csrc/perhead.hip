// Per-head position keys: the simplified MLA-style cache of "Multi-Head
// Latent Attention" (talalahmed.dev), "A concrete size comparison": each
// token keeps the latent c_t and one RoPE key per head, 256 + 16 x 32 = 768
// numbers.  Head i scores
//     s_{i,t} = scale (q~_i . c_t + R_m q^R_i . R_t k^R_{t,i})
// and the latent output is obar_i = sum_t alpha_{i,t} c_t, as in the shared
// layout; only the position key differs per head.
//
// Shape: 16 heads, d_c = 256, d_r = 32 (that page's example).  A cache row is
// [c_t | R_t k^R_{t,0} | ... | R_t k^R_{t,15}], 1536 bytes, every key stored
// already rotated to its own position.
//
// The position part is a block-diagonal contraction: seen as one 768-wide
// score, head i's query is [q~_i | 0 .. R_m q^R_i .. 0] with its position
// block at 256 + 32 i.  With d_r = 32 each position block is exactly one
// k-step of v_mfma_f32_16x16x32_bf16, so k-step j of the position part
// multiplies head j's query block and zeros for the other heads: the same
// MFMA stream as a dense 768-wide score, at 16 / 16 useful columns in the
// content steps and 1 / 16 in the position steps.  The kernel moves 1536
// bytes per token and does ~26 KFLOP per token on the MFMA pipe, so it is
// bound by HBM, and the wasted MFMA columns cost nothing measurable.
//
// Decode: a workgroup of 4 waves takes one (sequence, split) item, the same
// split plan and partial format as the shared-key decode kernel (so its
// merge kernel combines the splits).  Each 64-token page goes HBM ->
// registers -> LDS (the next page's 24 loads per thread are in flight while
// the current one is scored), then:
//   * scores: wave w takes 16 tokens (a row permutation chosen so that the
//     MFMA result lands in the layout the P.V product reads), 24 k-steps;
//   * softmax: per-head page max shared through LDS, running max and sum,
//     the accumulators rescaled per lane (each lane holds one head);
//   * P.V: O^T[col][head] += C^T[col][t] P^T[t][head]; wave w owns latent
//     columns 64 w .. 64 w + 63 of every head, the C^T operand comes from the
//     page in LDS by transpose reads, P^T from LDS.
#include "common.hpp"
#include "decode_items.hpp"

namespace mla {

namespace {

constexpr int kPhH = 16;                   // heads
constexpr int kPhDc = 256;                 // latent width
constexpr int kPhDr = 32;                  // position key width per head
constexpr int kPhRow = kPhDc + kPhH * kPhDr;  // 768 elements per cache row
constexpr int kPhStride = kPhRow + 8;      // LDS row stride (elements): 1552 bytes
constexpr int kPhChunks = kPhRow / 8;      // 16-byte chunks per row: 96
constexpr int kPhLoads = kPage * kPhChunks / 256;  // 16-byte loads per thread per page: 24
constexpr int kPhPStride = kPage + 8;      // P row stride (elements) in LDS
constexpr float kPhLn2 = 0.69314718055994530942f;
// Word 3 of a raw (untyped) buffer resource: 32-bit data format, no swizzle,
// no index addressing; loads past num_records return zeros.
constexpr int kPhBufferWord3 = 0x00020000;
static_assert(kPage * kPhChunks % 256 == 0, "a page must split evenly over the threads");
static_assert(kPhDr == 32, "one position block per 32-wide k-step");

template <bool F32W>
__global__ void __launch_bounds__(256, 1) perhead_decode_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[kPage * kPhStride];
  // softmax weights P^T of the page (with F32W, their lo terms follow)
  __shared__ __attribute__((aligned(16))) bf16_t pbuf[(F32W ? 2 : 1) * kPhH * kPhPStride];
  __shared__ float red[4][kPhH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15, q16 = lane >> 4;

  const int64_t item = xcd_local(blockIdx.x, gridDim.x);
  const DecodeItem it = find_decode_item(p, item);
  if (!it.ok || it.slot >= p.n_items) return;
  const int b = __builtin_amdgcn_readfirstlane(it.b);
  if (b >= p.num_seqs) return;
  const int key_end = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
  const int pages = (key_end + kPage - 1) / kPage;
  const int page_begin = __builtin_amdgcn_readfirstlane(it.s) * p.split_pages;
  const int page_end = min(pages, page_begin + p.split_pages);
  const bool final_out = !p.all_partials && __builtin_amdgcn_readfirstlane(it.n_s) == 1;
  const int slot = __builtin_amdgcn_readfirstlane(it.slot);

  // ---- query fragments (MFMA B operand: head r16, k = 8 q16 .. 8 q16 + 7 of a
  // 32-wide k-step).  Content: q~ of head r16, 8 k-steps.  Position: head r16's
  // rotated q^R (one k-step), used only in k-step r16 of the position part.
  // A float32 q_lat enters as hi = bf16(q) and lo = bf16(q - hi), two terms.
  bf16x8 qc_hi[kPhDc / 32], qc_lo[F32W ? kPhDc / 32 : 1];
  bf16x8 qr_hi, qr_lo;
  {
    const int64_t qrow = static_cast<int64_t>(b) * kPhH + r16;
    auto frag = [&](int k0, bf16x8& hi, bf16x8& lo) {
      if constexpr (F32W) {
        const float* q = static_cast<const float*>(p.q_lat) + qrow * (kPhDc + kPhDr) + k0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = q[e];
          const __bf16 h = static_cast<__bf16>(v);
          hi[e] = h;
          lo[e] = static_cast<__bf16>(v - static_cast<float>(h));
        }
      } else {
        hi = *reinterpret_cast<const bf16x8*>(static_cast<const bf16_t*>(p.q_lat) + qrow * (kPhDc + kPhDr) + k0);
        (void)lo;
      }
    };
#pragma unroll
    for (int ks = 0; ks < kPhDc / 32; ++ks) frag(ks * 32 + 8 * q16, qc_hi[ks], qc_lo[F32W ? ks : 0]);
    frag(kPhDc + 8 * q16, qr_hi, qr_lo);
  }
  const bf16x8 zero8 = {};

  // ---- page loads: thread tid moves chunks tid + 256 i (row c / 96, chunk c % 96)
  // through a raw buffer resource over the page's valid rows: one lane offset
  // for all 24 loads, and the hardware returns zeros past the sequence's end
  // (and for a page the table does not name), which keeps those slots out of
  // P.V even where P is 0.
  i32x4 ld[kPhLoads];
  auto page_id = [&](int pg) { return p.block_table[static_cast<int64_t>(b) * p.max_pages + pg]; };
  auto load_page = [&](int pg, int page) {
    page = __builtin_amdgcn_readfirstlane(page);
    const bool ok = page >= 0 && page < p.num_pages;
    const int valid = ok ? min(kPage, key_end - pg * kPage) : 0;
    const bf16_t* base = static_cast<const bf16_t*>(p.cache) + static_cast<int64_t>(ok ? page : 0) * kPage * kPhRow;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), 0, valid * kPhRow * 2, kPhBufferWord3);
#pragma unroll
    // nt: each page is read once, by one workgroup (2-3% faster at 64 x 4096)
    for (int i = 0; i < kPhLoads; ++i) ld[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, i * 4096, kCpolNt);
  };
  auto store_page = [&]() {
#pragma unroll
    for (int i = 0; i < kPhLoads; ++i) {
      const int c = tid + 256 * i;
      const int row = c / kPhChunks, ch = c % kPhChunks;
      *reinterpret_cast<i32x4*>(&tile[row * kPhStride + ch * 8]) = ld[i];
    }
  };

  // score rows of wave w: row r <-> token 32 (w >> 1) + 8 (r >> 2) + 4 (w & 1) + (r & 3),
  // so a lane's four results (rows 4 q16 .. 4 q16 + 3) and its partner wave's
  // four are the eight consecutive tokens 32 g + 8 q16 .. + 7 the P.V B operand holds
  const int g = wave >> 1, half = wave & 1;
  const int a_tok = 32 * g + 8 * (r16 >> 2) + 4 * half + (r16 & 3);  // token of this lane's A row
  const int d_tok0 = 32 * g + 8 * q16 + 4 * half;                    // token of this lane's result 0

  f32x4 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of the scaled log2 scores of head r16
  float l_run = 0.f;        // this lane's share of the sum of P of head r16

  // The block-table entry of the page after next is fetched with the next
  // page's loads, so no page waits on a table read of its own.
  int id_next = 0;
  if (page_begin < page_end) {
    const int id0 = page_id(page_begin);
    if (page_begin + 1 < page_end) id_next = page_id(page_begin + 1);
    load_page(page_begin, id0);
  }
  for (int pg = page_begin; pg < page_end; ++pg) {
    __syncthreads();  // every wave is done with the previous page
    store_page();
    if (pg + 1 < page_end) {  // in flight while this page is scored
      const int id = id_next;
      if (pg + 2 < page_end) id_next = page_id(pg + 2);
      load_page(pg + 1, id);
    }
    __syncthreads();

    // ---- scores S^T[token][head]
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16_t* arow = &tile[a_tok * kPhStride + 8 * q16];
#pragma unroll
    for (int ks = 0; ks < kPhDc / 32; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + ks * 32);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qc_hi[ks], s, 0, 0, 0);
      if constexpr (F32W) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qc_lo[ks], s, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kPhH; ++j) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + kPhDc + j * kPhDr);
      // The head index goes through an empty asm so that the selected operand
      // is formed here, four selects a step, rather than all sixteen hoisted
      // out of the page loop into 64 more registers.
      int jj = j;
      asm volatile("" : "+s"(jj));
      const bool own = r16 == jj;
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, own ? qr_hi : zero8, s, 0, 0, 0);
      if constexpr (F32W) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, own ? qr_lo : zero8, s, 0, 0, 0);
    }

    // ---- softmax over the page, head r16; tokens past the end are masked
    const int tok_base = pg * kPage + d_tok0;
    float x[4];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = tok_base + e < key_end ? s[e] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[e]);
    }
    mx = pair32_max(pair16_max(mx));
    if (q16 == 0) red[wave][r16] = mx;
    __syncthreads();
    const float page_max = fmaxf(fmaxf(red[0][r16], red[1][r16]), fmaxf(red[2][r16], red[3][r16]));
    const float m_new = fmaxf(m_run, page_max);  // finite: every page holds a visible token
    const float alpha = exp2f(m_run - m_new);    // 0 on the first page
    m_run = m_new;
    float pv[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pv[e] = exp2f(x[e] - m_new);
      psum += pv[e];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
    uint2 pk;
    pk.x = pack_bf16x2(pv[0], pv[1]);
    pk.y = pack_bf16x2(pv[2], pv[3]);
    *reinterpret_cast<uint2*>(&pbuf[r16 * kPhPStride + d_tok0]) = pk;
    if constexpr (F32W) {
      // lo terms: P - bf16(P), exact in float32, then rounded once
      float rest[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t word = e < 2 ? pk.x : pk.y;
        rest[e] = pv[e] - bf16_to_f32(static_cast<bf16_t>((e & 1) ? word >> 16 : word & 0xffffu));
      }
      uint2 pl;
      pl.x = pack_bf16x2(rest[0], rest[1]);
      pl.y = pack_bf16x2(rest[2], rest[3]);
      *reinterpret_cast<uint2*>(&pbuf[kPhH * kPhPStride + r16 * kPhPStride + d_tok0]) = pl;
    }
    __syncthreads();

    // ---- P.V: O^T[col][head] over the page's two 32-token k-steps
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const bf16x8 pb = *reinterpret_cast<const bf16x8*>(&pbuf[r16 * kPhPStride + 32 * kt + 8 * q16]);
      bf16x8 pbl;
      if constexpr (F32W) pbl = *reinterpret_cast<const bf16x8*>(&pbuf[(kPhH + r16) * kPhPStride + 32 * kt + 8 * q16]);
      const int t0 = 32 * kt + 8 * q16 + (r16 >> 2);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int col = wave * 64 + cb * 16 + 4 * (r16 & 3);
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(&tile[t0 * kPhStride + col]));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(&tile[(t0 + 4) * kPhStride + col]));
        bf16x8 a;
        __builtin_memcpy(&a, &lo, 8);
        __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
        oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, oacc[cb], 0, 0, 0);
        if constexpr (F32W) oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pbl, oacc[cb], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: l of head r16 over the four q16 lanes and the four waves
  const float l_wave = pair32_sum(pair16_sum(l_run));
  __syncthreads();
  if (q16 == 0) red[wave][r16] = l_wave;
  __syncthreads();
  const float l = (red[0][r16] + red[1][r16]) + (red[2][r16] + red[3][r16]);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t hrow = final_out ? static_cast<int64_t>(b) * kPhH + r16 : static_cast<int64_t>(slot) * kPhH + r16;
  float* out = (final_out ? static_cast<float*>(p.out_latent) : p.ws_o) + hrow * kPhDc;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    *reinterpret_cast<f32x4*>(out + wave * 64 + cb * 16 + 4 * q16) =
        f32x4{oacc[cb][0] * inv, oacc[cb][1] * inv, oacc[cb][2] * inv, oacc[cb][3] * inv};
  if (wave == 0 && q16 == 0) {
    const float lse_v = l > 0.f ? (m_run + log2f(l)) * kPhLn2 : -INFINITY;
    if (final_out) {
      if (p.lse != nullptr) p.lse[hrow] = lse_v;
    } else {
      p.ws_lse[hrow] = lse_v;
    }
  }
}

// Cache rows [c_t | R_t k^R_{t,0} | ... | R_t k^R_{t,H-1}]: one wave per row.
// Angles and rotation in float64, rounded once (as the shared-key write).
__global__ void __launch_bounds__(256) perhead_cache_write_kernel(RopeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (m >= p.n_kv) return;
  const int b = p.kv_seq[m];
  const int pos = p.kv_pos[m];
  if (b < 0 || b >= p.num_seqs || pos < 0) return;
  const int lp = pos / kPage;
  if (lp >= p.max_pages) return;
  const int page = p.block_table[static_cast<int64_t>(b) * p.max_pages + lp];
  if (page < 0 || page >= p.num_pages) return;
  const int width = p.d_latent + p.n_heads * p.d_rope;
  bf16_t* dst = static_cast<bf16_t*>(p.cache) + (static_cast<int64_t>(page) * kPage + pos % kPage) * width;
  const bf16_t* lat = static_cast<const bf16_t*>(p.kv_latent) + m * p.d_latent;
  for (int c = lane; c < p.d_latent; c += 64) dst[c] = lat[c];
  const bf16_t* kr = static_cast<const bf16_t*>(p.k_rope) + m * p.n_heads * p.d_rope;
  const int half = p.d_rope / 2;
  for (int q = lane; q < p.n_heads * half; q += 64) {
    const int h = q / half, j = q % half;
    double sn, cs;
    sincos(static_cast<double>(pos) * p.theta[j], &sn, &cs);
    const double x0 = bf16_to_f32(kr[h * p.d_rope + 2 * j]), x1 = bf16_to_f32(kr[h * p.d_rope + 2 * j + 1]);
    *reinterpret_cast<uint32_t*>(dst + p.d_latent + h * p.d_rope + 2 * j) =
        pack_bf16x2(static_cast<float>(x0 * cs - x1 * sn), static_cast<float>(x0 * sn + x1 * cs));
  }
}

}  // namespace

hipError_t launch_perhead_decode(const AttnParams& p, hipStream_t s) {
  if (p.n_items == 0) return hipSuccess;
  if (p.n_heads != kPhH || p.d_latent != kPhDc || p.d_rope != kPhDr) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.n_items));
  if (p.f32w)
    hipLaunchKernelGGL(perhead_decode_kernel<true>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(perhead_decode_kernel<false>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_perhead_cache_write(const RopeParams& p, hipStream_t s) {
  if (p.n_kv == 0) return hipSuccess;
  hipLaunchKernelGGL(perhead_cache_write_kernel, dim3(static_cast<unsigned>((p.n_kv + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
