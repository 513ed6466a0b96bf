// paged_decode_attn kernels for gfx950: split-K (flash-decoding) decode
// attention over a paged K/V cache held as e4m3 (or BF16), with the page-tag
// check done before any page's contents are used.
//
// What is computed (source pages: "Cloudflare tối ưu hóa Kimi và GLM trên
// Workers AI", section "Lượng tử hóa KV cache" -- the attention kernel reads
// an FP8 e4m3 cache and converts values as it reads them; "ترفندهای کلادفلر
// برای جا دادن مدل‌های غول‌پیکر تو GPU", third technique, and "Tối ưu hóa mô
// hình AI quy mô lớn", section "Bảo vệ tính toàn vẹn của KV Cache" -- each
// page carries a tag that changes on reallocation, checked before the page
// is read, a mismatch aborting the request):
//
//   out[b][h] = sum_t softmax_t(scale * <q[b][h], k_t>) v_t
//
// over the L = seq_lens[b] tokens of KV head h / G, read through the page
// table; nothing is written for a sequence whose pages fail the check.
//
// Kernels of one call
// -------------------
// 1. With tags on, a page check (check_block in page_check.hpp: one block per
//    1024 page-table slots of a sequence) checks every used page slot of
//    every sequence -- page id in range, tag equal to the expected tag -- and
//    the length.  It is its own kernel in paged_decode_attn and shares the
//    first kernel of a decode step with the append's blocks.
// 2. decode_kernel writes the abort flags and streams K/V for the
//    sequences that passed.  With tags off no check ran: the schedule checks
//    the lengths, and every round of page ids a wave loads is range-checked
//    before any of its pages is read (a failing piece stops and reports).
// 3. merge_kernel combines the partial results of split segments and adds
//    the bits of pieces that failed the range check.
// With tags on the check comes first so that an aborted sequence costs 12
// bytes per page (id, tag, expected tag) instead of its K/V, and is left out
// of the work partition, which keeps the shares of the other sequences
// balanced.
//
// Work decomposition
// ------------------
// The batch's work is the flattened list of (sequence, KV head, 64-token
// tile) triples of the sequences that passed the check.  A 1-D grid of
// blocks of 4 independent waves cuts it into equal contiguous shares, one per wave (see "The balanced schedule"), so
// every wave streams the same number of bytes whatever the length mix and
// long sequences are split across waves (flash-decoding).  A wave keeps an
// online-softmax state (running max m, sum l, unnormalized acc) per piece
// of one (sequence, KV head); a piece that is a whole segment is finished in
// registers, a partial piece is published to the workspace and the merge
// kernel combines the partials (log-sum-exp) and writes the output.  No
// wave ever waits for another.

// Per wave and tile (MFMA family, group of 5..16 query heads per KV head):
//   * K rows: lane l loads a quarter of one token's row (bytes of dims
//     [q*D/4, (q+1)*D/4), q = l/16) for 4 token blocks; 16 lanes cover one
//     full row, so every load instruction reads whole 128-byte lines.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 dims of
//     K (e4m3 -> bf16 exact in registers), B = 32 dims x 16 query heads.  The
//     dims a lane contributes at each k-step are relabelled consistently in
//     A and B, which is what lets a lane read 32 contiguous bytes.
//   * Tokens are relabelled so that the C layout of S^T (lane l holds head
//     l%16 for 4 tokens) is exactly the B layout P^T needs for PV -- no data
//     moves between lanes between the two products.
//   * O^T = V^T P^T with v_mfma_f32_16x16x32_f16 (FP8: e4m3 -> f16 exact,
//     P rounded to f16) or _bf16 (BF16 cache).  FP8: the V tile is copied
//     global -> LDS by global_load_lds_dwordx4 and read back transposed by
//     ds_read_b64_tr_b8.  BF16: lane l loads 16 tokens x D/16 contiguous
//     dims of V and a half-word transpose in registers (v_perm_b32) builds
//     the A operand.  The accumulator layout puts head l%16 in lane l, the
//     same lane that owns its softmax state.
//   * The K/V stream is loaded non-temporal (read once per call).
//   * Softmax max/sum across the 4 lane groups: wave shuffles.
// VALU family (groups of 1..4): lane = (token slot, dim chunk); dot products
// with v_dot2_f32_bf16 and fp32 FMA, octet sums through DPP.
//
// Scales: k_scale * softmax_scale * log2(e) multiplies the fp32 scores and
// v_scale the final output, so dequantization itself adds no rounding.
#include "common.hpp"
#include "internal.hpp"
#include "page_check.hpp"

namespace fp8kv {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// ------------------------------------------------------------------------
// Geometry of one element type / head size.
// ------------------------------------------------------------------------
template <int KV, int D>
struct Geo {
  static constexpr int ESZ = KV == 0 ? 1 : 2;   // bytes per cache element
  static constexpr int ROW = D * ESZ;           // bytes per (token, KV head) row
  // MFMA family
  static constexpr int KSTEPS = D / 32;         // QK k-steps of 32 dims
  static constexpr int NB = D / 16;             // PV output blocks of 16 dims
  static constexpr int KQ = D / 4 * ESZ;        // K bytes per lane per token (a quarter row)
  static constexpr int KQV = KQ / 16;           // 16-byte loads per quarter row
  static constexpr int VW = NB * ESZ / 4;       // V words (4 bytes) per lane per token
  // VALU family
  static constexpr int DC = D / 8;              // dims per lane
  static constexpr int CW = DC * ESZ / 4;       // words per lane per token
};

// Cache-policy operand of global_load_lds for a non-temporal load (the
// instruction's nt bit on gfx950).
constexpr int kCpolNonTemporal = 2;
template <int KV>
constexpr bool kNonTemporalK = KV == 0;  // see load_words

// Load N consecutive 4-byte words with the widest aligned vector loads.
// NT: non-temporal.  The K/V stream is read once per call, and loading it
// non-temporal (V always -- also its FP8 copy to LDS -- and K from an FP8
// cache) streams it markedly faster: at batch 32, 68% -> 75% of 8 TB/s for
// FP8 and 71% -> 79% for BF16.  A BF16 cache's K loads stay cached: each
// lane's 64-byte quarter row takes four 16-byte loads, and marked
// non-temporal they ran at 62%.
template <int N, bool NT = false>
__device__ __forceinline__ void load_words(const uint8_t* src, uint32_t* dst) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const u32x4_t* a = reinterpret_cast<const u32x4_t*>(src + 4 * i);
      u32x4_t x;
      if constexpr (NT)
        x = __builtin_nontemporal_load(a);
      else
        x = *a;
      dst[i] = x[0]; dst[i + 1] = x[1]; dst[i + 2] = x[2]; dst[i + 3] = x[3];
    }
  } else if constexpr (N == 2) {
    const u32x2_t* a = reinterpret_cast<const u32x2_t*>(src);
    u32x2_t x;
    if constexpr (NT)
      x = __builtin_nontemporal_load(a);
    else
      x = *a;
    dst[0] = x[0]; dst[1] = x[1];
  } else {
    static_assert(N == 1, "unsupported word count");
    const uint32_t* a = reinterpret_cast<const uint32_t*>(src);
    if constexpr (NT)
      dst[0] = __builtin_nontemporal_load(a);
    else
      dst[0] = *a;
  }
}

// ------------------------------------------------------------------------
// Page walk: the wave's page list for a round of its tiles.
// ------------------------------------------------------------------------
struct PageRound {
  int pid;       // lane j: physical page of wave page j (a safe substitute where unused)
  int log2ps;
  int ppt_log2;  // log2(pages per tile) when pages are smaller than a tile, else 0
};

// Physical page holding 16-token group `grp16` (0..3) of the round's tile `i`.
__device__ __forceinline__ int page_of(const PageRound& pr, int i, int grp16) {
  if (pr.log2ps >= 6) return __builtin_amdgcn_readlane(pr.pid, i);
  return __shfl(pr.pid, (i << pr.ppt_log2) + (grp16 >> (pr.log2ps - 4)));
}

__device__ __forceinline__ const uint8_t* row_ptr(const uint8_t* cache, int pid, int g, int hkv,
                                                  int log2ps, int slot, int row_bytes) {
  return cache + ((((int64_t)pid * hkv + g) << log2ps) + slot) * (int64_t)row_bytes;
}

// ------------------------------------------------------------------------
// MFMA family.
// ------------------------------------------------------------------------
template <int KV, int D>
struct MfmaTile {
  using G_ = Geo<KV, D>;
  uint32_t k[4][G_::KQ / 4];   // token block bb: this lane's quarter row
  uint32_t v[16][G_::VW];      // 16 tokens: this lane's D/16 dims
};
// FP8 cache: only K is held in registers; V streams through LDS (see below).
template <int D>
struct MfmaTile<0, D> {
  uint32_t k[4][Geo<0, D>::KQ / 4];
};

template <int KV, int D>
struct MfmaState {
  float m, l;
  f32x4_t acc[Geo<KV, D>::NB];
  bf16x8_t q[Geo<KV, D>::KSTEPS];
};

template <int KV, int D>
__device__ __forceinline__ void mfma_load_k(MfmaTile<KV, D>& t, const uint8_t* kp) {
  using G_ = Geo<KV, D>;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) load_words<G_::KQ / 4, kNonTemporalK<KV>>(kp + bb * 4 * G_::ROW, t.k[bb]);
}
template <int KV, int D>
__device__ __forceinline__ void mfma_load_v(MfmaTile<KV, D>& t, const uint8_t* vp) {
  using G_ = Geo<KV, D>;
  if constexpr (KV != 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) load_words<G_::VW, true>(vp + i * G_::ROW, t.v[i]);
  }
}

// S^T for the tile's 64 tokens: s[bb][r] = score of token 16*(lane/16) + 4*bb + r
// for query head lane%16 (unscaled).
template <int KV, int D>
__device__ __forceinline__ void mfma_qk(const MfmaTile<KV, D>& t, const MfmaState<KV, D>& st, f32x4_t s[4]) {
  using G_ = Geo<KV, D>;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < G_::KSTEPS; ++kk) {
      bf16x8_t a;
      if constexpr (KV == 0) {
        a = e4m3x8_to_bf16x8(t.k[bb][2 * kk], t.k[bb][2 * kk + 1]);
      } else {
        u32x4_t w = {t.k[bb][4 * kk], t.k[bb][4 * kk + 1], t.k[bb][4 * kk + 2], t.k[bb][4 * kk + 3]};
        a = __builtin_bit_cast(bf16x8_t, w);
      }
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, st.q[kk], c, 0, 0, 0);
    }
    s[bb] = c;
  }
}

// Online softmax update for the tile and O^T += V^T P^T.
template <int KV, int D>
__device__ __forceinline__ void mfma_softmax_pv(MfmaTile<KV, D>& t, MfmaState<KV, D>& st, f32x4_t s[4],
                                                int valid, float scale_log2, int lane) {
  using G_ = Geo<KV, D>;
  const int vg = lane >> 4;
  float mt = kNegInf;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = s[bb][r] * scale_log2;
      if (valid < kTileTokens && 16 * vg + 4 * bb + r >= valid) x = kNegInf;
      s[bb][r] = x;
      mt = __builtin_fmaxf(mt, x);
    }
  mt = xor_max(mt, 16);
  mt = xor_max(mt, 32);
  const float m_new = __builtin_fmaxf(st.m, mt);
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
  st.m = m_new;
  st.l *= alpha;
#pragma unroll
  for (int nb = 0; nb < G_::NB; ++nb) st.acc[nb] *= alpha;
  float pr[4][4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[bb][r] = fast_exp2(s[bb][r] - m_use);
      st.l += pr[bb][r];
    }

  // Rows past the sequence end may hold anything (even NaN codes): zero them.
  if (valid < kTileTokens) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (16 * vg + i >= valid)
#pragma unroll
        for (int w = 0; w < G_::VW; ++w) t.v[i][w] = 0u;
  }

#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if constexpr (KV == 0) {
      // B = P^T (f16): slots 0..3 = tokens 8ks+0..3, 4..7 = tokens 8ks+4..7 of this lane group
      f16x8_t bop;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bop[r] = (_Float16)pr[2 * ks][r];
        bop[4 + r] = (_Float16)pr[2 * ks + 1][r];
      }
      // A = V^T: byte-transpose 8 tokens x (4 dims per word) -> per dim 8 tokens
#pragma unroll
      for (int w = 0; w < G_::VW; ++w) {
        uint32_t lo[4], hi[4];
        transpose4x4_bytes(t.v[8 * ks + 0][w], t.v[8 * ks + 1][w], t.v[8 * ks + 2][w], t.v[8 * ks + 3][w],
                           lo[0], lo[1], lo[2], lo[3]);
        transpose4x4_bytes(t.v[8 * ks + 4][w], t.v[8 * ks + 5][w], t.v[8 * ks + 6][w], t.v[8 * ks + 7][w],
                           hi[0], hi[1], hi[2], hi[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x8_t aop = e4m3x8_to_f16x8(lo[e], hi[e]);
          st.acc[4 * w + e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, st.acc[4 * w + e], 0, 0, 0);
        }
      }
    } else {
      bf16x8_t bop;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bop[r] = (__bf16)pr[2 * ks][r];
        bop[4 + r] = (__bf16)pr[2 * ks + 1][r];
      }
      // word w of a token holds dims (2w, 2w+1); pair tokens for each dim
#pragma unroll
      for (int w = 0; w < G_::VW; ++w) {
        u32x4_t a0, a1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a0[j] = pair_lo16(t.v[8 * ks + 2 * j][w], t.v[8 * ks + 2 * j + 1][w]);
          a1[j] = pair_hi16(t.v[8 * ks + 2 * j][w], t.v[8 * ks + 2 * j + 1][w]);
        }
        st.acc[2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), bop,
                                                                st.acc[2 * w], 0, 0, 0);
        st.acc[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), bop,
                                                                    st.acc[2 * w + 1], 0, 0, 0);
      }
    }
  }
}

// ------------------------------------------------------------------------
// FP8 V through LDS.
//
// A 64-token V tile of one (page, KV head) is 64 rows of D bytes.  Each wave
// copies its next tile global -> LDS with global_load_lds_dwordx4 (lane j of
// an instruction lands at LDS base + 16 j, so 1 KiB per instruction and no
// VGPRs in flight), then reads it back with ds_read_b64_tr_b8, which
// transposes 8x16-byte blocks across each 16-lane group: lane j receives byte
// j of 8 consecutive 16-byte rows -- exactly the V^T operand of the PV MFMA
// (one dim, 8 tokens).  16-byte chunks are XOR-swizzled with the row index
// so that the 8 rows of a read fall in different LDS banks.
//
// The compiler waits for every outstanding LDS DMA before any LDS read, so
// the order per tile is: read tile i out of LDS, then start the copy of tile
// i+1 into the same buffer, then compute tile i.
// ------------------------------------------------------------------------
typedef int v2i_t __attribute__((ext_vector_type(2)));
#define FP8KV_LDS(ptr) ((__attribute__((address_space(3))) void*)(ptr))

// Physical page of 16-token group `grp16` of the round's tile `i`, for a
// wave-uniform group (scalar read of the page list).
__device__ __forceinline__ int page_of_uniform(const PageRound& pr, int i, int grp16) {
  const int idx = pr.log2ps >= 6 ? i : (i << pr.ppt_log2) + (grp16 >> (pr.log2ps - 4));
  return __builtin_amdgcn_readlane(pr.pid, idx);
}

template <int D>
__device__ __forceinline__ void v_tile_to_lds(const DecodeParams& p, const PageRound& pr, int i, int tile_abs, int g,
                                              int lane, uint8_t* stage) {
  constexpr int ROW = Geo<0, D>::ROW;       // bytes per token row
  constexpr int CH = ROW / 16;              // 16-byte chunks per row
  constexpr int RPI = 64 / CH;              // rows per DMA instruction (1 KiB)
  const int ps_mask = (1 << pr.log2ps) - 1;
  const int base_tok = tile_abs << 6;
  const int row_in = lane / CH, c = lane % CH;
#pragma unroll
  for (int m = 0; m < kTileTokens / RPI; ++m) {
    const int t = m * RPI + row_in;                       // token within the tile
    const int pid = page_of_uniform(pr, i, (m * RPI) >> 4);
    const uint8_t* src = row_ptr(p.v_cache, pid, g, p.num_kv_heads, pr.log2ps, (base_tok + t) & ps_mask, ROW) +
                         16 * (c ^ (t & (CH - 1)));
    __builtin_amdgcn_global_load_lds(src, FP8KV_LDS(stage + m * 1024), 16, 0, kCpolNonTemporal);
  }
}

// vt[ks][nb]: 8 e4m3 codes of dim 16*nb + lane%16 for tokens 16*(lane/16) + 8*ks + 0..7.
template <int D>
__device__ __forceinline__ void v_tile_from_lds(const uint8_t* stage, int lane, v2i_t (&vt)[2][Geo<0, D>::NB]) {
  constexpr int ROW = Geo<0, D>::ROW;
  constexpr int CH = ROW / 16;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int t = 16 * (lane >> 4) + 8 * ks + ((lane & 15) >> 1);
#pragma unroll
    for (int nb = 0; nb < Geo<0, D>::NB; ++nb) {
      const uint8_t* a = stage + t * ROW + 16 * (nb ^ (t & (CH - 1))) + 8 * (lane & 1);
      vt[ks][nb] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i_t*)(a));
    }
  }
}

// Online softmax update and O^T += V^T P^T for an FP8 tile whose V operands
// came from LDS (vt); same score layout as mfma_softmax_pv.
template <int D>
__device__ __forceinline__ void mfma_softmax_pv_lds(MfmaState<0, D>& st, f32x4_t s[4], v2i_t (&vt)[2][Geo<0, D>::NB],
                                                    int valid, float scale_log2, int lane) {
  using G_ = Geo<0, D>;
  const int vg = lane >> 4;
  float mt = kNegInf;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = s[bb][r] * scale_log2;
      if (valid < kTileTokens && 16 * vg + 4 * bb + r >= valid) x = kNegInf;
      s[bb][r] = x;
      mt = __builtin_fmaxf(mt, x);
    }
  mt = xor_max(mt, 16);
  mt = xor_max(mt, 32);
  const float m_new = __builtin_fmaxf(st.m, mt);
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
  st.m = m_new;
  st.l *= alpha;
#pragma unroll
  for (int nb = 0; nb < G_::NB; ++nb) st.acc[nb] *= alpha;
  f16x8_t bop[2];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = fast_exp2(s[bb][r] - m_use);
      st.l += e;
      bop[bb >> 1][4 * (bb & 1) + r] = (_Float16)e;
    }
  // Rows past the sequence end may hold anything (even NaN codes): zero them.
  if (valid < kTileTokens) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int t0 = 16 * vg + 8 * ks;  // token of byte 0
      const int n_ok = min(max(valid - t0, 0), 8);
      const uint64_t keep = n_ok >= 8 ? ~0ull : ((1ull << (8 * n_ok)) - 1ull);
#pragma unroll
      for (int nb = 0; nb < G_::NB; ++nb) {
        vt[ks][nb].x &= (int)(uint32_t)keep;
        vt[ks][nb].y &= (int)(uint32_t)(keep >> 32);
      }
    }
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int nb = 0; nb < G_::NB; ++nb) {
      const f16x8_t aop = e4m3x8_to_f16x8((uint32_t)vt[ks][nb].x, (uint32_t)vt[ks][nb].y);
      st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[ks], st.acc[nb], 0, 0, 0);
    }
}

// ------------------------------------------------------------------------
// VALU family.
// ------------------------------------------------------------------------
template <int KV, int D>
struct ValuTile {
  uint32_t k[8][Geo<KV, D>::CW];
  uint32_t v[8][Geo<KV, D>::CW];
};

template <int KV, int D, int GM>
struct ValuState {
  float m[GM], l[GM];
  float acc[GM][Geo<KV, D>::DC];
  uint32_t q2[GM][Geo<KV, D>::DC / 2];  // bf16 pairs of the query
};

template <int KV, int D>
__device__ __forceinline__ void valu_load(ValuTile<KV, D>& t, const uint8_t* kp, const uint8_t* vp) {
#pragma unroll
  for (int u = 0; u < 8; ++u) load_words<Geo<KV, D>::CW, kNonTemporalK<KV>>(kp + u * Geo<KV, D>::ROW, t.k[u]);
#pragma unroll
  for (int u = 0; u < 8; ++u) load_words<Geo<KV, D>::CW, true>(vp + u * Geo<KV, D>::ROW, t.v[u]);
}

// bf16 pairs of one token's DC dims
template <int KV, int D>
__device__ __forceinline__ void valu_pairs(const uint32_t* w, uint32_t* out) {
  if constexpr (KV == 0) {
#pragma unroll
    for (int i = 0; i < Geo<KV, D>::CW; ++i) {
      out[2 * i] = e4m3x2_to_bf16x2<false>(w[i]);
      out[2 * i + 1] = e4m3x2_to_bf16x2<true>(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < Geo<KV, D>::CW; ++i) out[i] = w[i];
  }
}

template <int KV, int D, int GM>
__device__ __forceinline__ void valu_qk(const ValuTile<KV, D>& t, const ValuState<KV, D, GM>& st,
                                        float s[8][GM]) {
  constexpr int DC = Geo<KV, D>::DC;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    uint32_t kp[DC / 2];
    valu_pairs<KV, D>(t.k[u], kp);
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < DC / 2; ++i)
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, st.q2[h][i]),
                                            __builtin_bit_cast(bf16x2_t, kp[i]), a, false);
      s[u][h] = octet_sum(a);
    }
  }
}

template <int KV, int D, int GM>
__device__ __forceinline__ void valu_softmax_pv(ValuTile<KV, D>& t, ValuState<KV, D, GM>& st, float s[8][GM],
                                                int valid, float scale_log2, int lane) {
  constexpr int DC = Geo<KV, D>::DC;
  const int ts = lane >> 3;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    float mt = kNegInf;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float x = s[u][h] * scale_log2;
      if (valid < kTileTokens && 8 * ts + u >= valid) x = kNegInf;
      s[u][h] = x;
      mt = __builtin_fmaxf(mt, x);
    }
    const float m_new = __builtin_fmaxf(st.m[h], mt);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(st.m[h] - m_use);
    st.m[h] = m_new;
    st.l[h] *= alpha;
#pragma unroll
    for (int i = 0; i < DC; ++i) st.acc[h][i] *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s[u][h] = fast_exp2(s[u][h] - m_use);
      st.l[h] += s[u][h];
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float vf[DC];
    if constexpr (KV == 0) {
#pragma unroll
      for (int i = 0; i < Geo<KV, D>::CW; ++i) e4m3x4_to_f32(t.v[u][i], vf + 4 * i);
    } else {
#pragma unroll
      for (int i = 0; i < Geo<KV, D>::CW; ++i) {
        vf[2 * i] = bf16_bits_to_f32(t.v[u][i] & 0xFFFFu);
        vf[2 * i + 1] = __builtin_bit_cast(float, t.v[u][i] & 0xFFFF0000u);
      }
    }
    if (valid < kTileTokens && 8 * ts + u >= valid) {
#pragma unroll
      for (int i = 0; i < DC; ++i) vf[i] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
      for (int i = 0; i < DC; ++i) st.acc[h][i] = __builtin_fmaf(s[u][h], vf[i], st.acc[h][i]);
  }
}

// ------------------------------------------------------------------------
// One wave: walk its consecutive tiles of one (sequence, KV head), checking
// the pages of each round before any of their contents are used.
// ------------------------------------------------------------------------
template <int KV, int D, int GM, bool MFMA>
struct WaveState;
template <int KV, int D, int GM>
struct WaveState<KV, D, GM, true> { using T = MfmaState<KV, D>; using Tile = MfmaTile<KV, D>; };
template <int KV, int D, int GM>
struct WaveState<KV, D, GM, false> { using T = ValuState<KV, D, GM>; using Tile = ValuTile<KV, D>; };

template <int KV, int D, int GM, bool MFMA>
__device__ __forceinline__ void tile_pointers(const DecodeParams& p, const PageRound& pr, int i, int tile_abs,
                                              int g, int lane, const uint8_t*& kp, const uint8_t*& vp) {
  using G_ = Geo<KV, D>;
  const int ps_mask = (1 << pr.log2ps) - 1;
  const int base_tok = tile_abs << 6;
  if constexpr (MFMA) {
    const int kg = (lane & 15) >> 2;
    const int ktok = 16 * kg + (lane & 3);
    const int vg = lane >> 4;
    const int kpid = page_of(pr, i, kg);
    const int vpid = page_of(pr, i, vg);
    kp = row_ptr(p.k_cache, kpid, g, p.num_kv_heads, pr.log2ps, (base_tok + ktok) & ps_mask, G_::ROW) +
         (lane >> 4) * G_::KQ;
    vp = row_ptr(p.v_cache, vpid, g, p.num_kv_heads, pr.log2ps, (base_tok + 16 * vg) & ps_mask, G_::ROW) +
         (lane & 15) * (G_::VW * 4);
  } else {
    const int ts = lane >> 3;
    const int pid = page_of(pr, i, ts >> 1);
    const int off = (lane & 7) * (G_::CW * 4);
    kp = row_ptr(p.k_cache, pid, g, p.num_kv_heads, pr.log2ps, (base_tok + 8 * ts) & ps_mask, G_::ROW) + off;
    vp = row_ptr(p.v_cache, pid, g, p.num_kv_heads, pr.log2ps, (base_tok + 8 * ts) & ps_mask, G_::ROW) + off;
  }
}

template <int KV, int D, int GM, bool MFMA>
__device__ __forceinline__ void load_tile(typename WaveState<KV, D, GM, MFMA>::Tile& t, const uint8_t* kp,
                                          const uint8_t* vp) {
  if constexpr (MFMA) {
    mfma_load_k<KV, D>(t, kp);
    mfma_load_v<KV, D>(t, vp);
  } else {
    valu_load<KV, D>(t, kp, vp);
  }
}

template <int KV, int D, int GM, bool MFMA>
__device__ __forceinline__ void compute_tile(typename WaveState<KV, D, GM, MFMA>::Tile& t,
                                             typename WaveState<KV, D, GM, MFMA>::T& st, int valid,
                                             float scale_log2, int lane) {
  if constexpr (MFMA) {
    f32x4_t s[4];
    mfma_qk<KV, D>(t, st, s);
    mfma_softmax_pv<KV, D>(t, st, s, valid, scale_log2, lane);
  } else {
    float s[8][GM];
    valu_qk<KV, D, GM>(t, st, s);
    valu_softmax_pv<KV, D, GM>(t, st, s, valid, scale_log2, lane);
  }
}

// Returns false (and stops) if a round's page ids include one outside
// [0, num_pages): no page of that round is read.  With tags on the page
// check already excluded such sequences, so this never fails then.
template <int KV, int D, int GM, bool MFMA>
__device__ __forceinline__ bool run_wave(const DecodeParams& p, int b, int g, int L, int first_tile, int n_wave_tiles,
                                         typename WaveState<KV, D, GM, MFMA>::T& st, int lane, uint8_t* vstage) {
  constexpr bool kVlds = MFMA && KV == 0;  // FP8 V streams through LDS
  using Tile = typename WaveState<KV, D, GM, MFMA>::Tile;
  const int log2ps = p.log2_page_size;
  const int ppt_log2 = log2ps < 6 ? 6 - log2ps : 0;
  const int round_tiles = 64 >> ppt_log2;
  const int n_pages_b = (L + (1 << log2ps) - 1) >> log2ps;
  const int64_t pt_row = (int64_t)b * p.max_pages;

  for (int r0 = 0; r0 < n_wave_tiles; r0 += round_tiles) {
    const int rt = min(round_tiles, n_wave_tiles - r0);
    // lane j -> wave page j of this round
    const int jt = lane >> ppt_log2;
    const int tile_j = first_tile + (r0 + jt);
    const int lp = log2ps < 6 ? (tile_j << ppt_log2) + (lane & ((1 << ppt_log2) - 1)) : (tile_j << 6) >> log2ps;
    const bool used = jt < rt && lp < n_pages_b;
    const int pid = used ? p.page_table[pt_row + lp] : 0;
    if (__ballot(used && (pid < 0 || pid >= p.num_pages)) != 0) return false;
    PageRound pr;
    pr.log2ps = log2ps;
    pr.ppt_log2 = ppt_log2;
    // Slots past the sequence's last page (only in its last tile) borrow the
    // tile's first page, which always exists; their rows are masked.
    const int first_pid = __shfl(pid, lane & ~((1 << ppt_log2) - 1));
    pr.pid = used ? pid : first_pid;

    Tile ta, tb;
    const uint8_t *kp, *vp;
    tile_pointers<KV, D, GM, MFMA>(p, pr, 0, first_tile + r0, g, lane, kp, vp);
    load_tile<KV, D, GM, MFMA>(ta, kp, vp);
    if constexpr (kVlds) v_tile_to_lds<D>(p, pr, 0, first_tile + r0, g, lane, vstage);

    if constexpr (kVlds) {
      // Per tile i: V(i) out of LDS; start V(i+1) into LDS; QK(i) from the K
      // registers; then start K(i+1) into those registers; softmax + PV(i).
      // Both next-tile streams are in flight while tile i is computed, and the
      // next iteration's LDS read waits for them (the compiler waits for all
      // LDS copies before an LDS read).  The last iteration still issues both
      // loads, so that no load sits under a condition, but computes their
      // addresses with lane index 0 in every lane: a few cache lines of the
      // round's last tile instead of the whole tile again.
      const float sl = p.qk_scale_log2;
      v2i_t vt[2][Geo<0, D>::NB];
      for (int i = 0; i < rt; ++i) {
        const int t0 = first_tile + (r0 + i);
        const int n1 = min(i + 1, rt - 1);
        const int pl = lane & (i + 1 < rt ? 63 : 0);  // lane index for the prefetch addresses
        v_tile_from_lds<D>(vstage, lane, vt);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): tile i is out of LDS before it is overwritten
        __builtin_amdgcn_sched_barrier(0);
        v_tile_to_lds<D>(p, pr, n1, first_tile + (r0 + n1), g, pl, vstage);
        f32x4_t sc[4];
        mfma_qk<KV, D>(ta, st, sc);
        __builtin_amdgcn_sched_barrier(0);
        tile_pointers<KV, D, GM, MFMA>(p, pr, n1, first_tile + (r0 + n1), g, pl, kp, vp);
        mfma_load_k<KV, D>(ta, kp);
        mfma_softmax_pv_lds<D>(st, sc, vt, min(L - (t0 << 6), kTileTokens), sl, lane);
      }
      __builtin_amdgcn_s_waitcnt(0);  // the last (redundant) copy has landed before LDS is reused
    } else {
    // Tile i is computed while tile i+1 loads.  The prefetch is issued on
    // every iteration: a prefetch under a condition would make the compiler
    // wait for it inside the current tile's math, serializing the pipeline.
    // Past the round's last tile its addresses use lane index 0 in every
    // lane (a few cache lines, results unused).
    const float sl = p.qk_scale_log2;
    for (int i = 0; i < rt; i += 2) {
      const int n1 = min(i + 1, rt - 1);
      tile_pointers<KV, D, GM, MFMA>(p, pr, n1, first_tile + (r0 + n1), g, lane & (i + 1 < rt ? 63 : 0), kp, vp);
      load_tile<KV, D, GM, MFMA>(tb, kp, vp);
      const int t0 = first_tile + (r0 + i);
      compute_tile<KV, D, GM, MFMA>(ta, st, min(L - (t0 << 6), kTileTokens), sl, lane);
      if (i + 1 >= rt) break;
      const int n2 = min(i + 2, rt - 1);
      tile_pointers<KV, D, GM, MFMA>(p, pr, n2, first_tile + (r0 + n2), g, lane & (i + 2 < rt ? 63 : 0), kp, vp);
      load_tile<KV, D, GM, MFMA>(ta, kp, vp);
      compute_tile<KV, D, GM, MFMA>(tb, st, min(L - ((t0 + 1) << 6), kTileTokens), sl, lane);
    }
    }
  }
  return true;
}

// ------------------------------------------------------------------------
// Leaving a piece: a wave's state -> output rows or a published partial.
//
// MFMA family: lane l owns head l%16 and, for accumulator block nb and row
// r, head-dim index acc_dim(nb, r, l); its running sum l is split over the 4
// lane groups.  VALU family: after a merge across token slots, lanes 0..7
// own dims [8*lane .. ) of every head.
// ------------------------------------------------------------------------
template <int KV, int D>
__device__ __forceinline__ int acc_dim(int nb, int r, int lane) {
  // FP8 (V^T read from LDS): dim 16*nb + 4*(lane/16) + r
  // BF16 (V^T built in registers): dim NB*(4*(lane/16) + r) + nb
  return KV == 0 ? 16 * nb + 4 * (lane >> 4) + r : Geo<KV, D>::NB * (4 * (lane >> 4) + r) + nb;
}

__device__ __forceinline__ void store_bf16(uint16_t* dst, float x) { *dst = (uint16_t)f32_to_bf16_bits(x); }

template <int KV, int D>
__device__ __forceinline__ void wave_output(MfmaState<KV, D>& st, const DecodeParams& p, int64_t out_row0, int lane) {
  float l = xor_sum(st.l, 16);
  l = xor_sum(l, 32);
  const int h = lane & 15;
  if (h < p.group) {
    const float inv = p.v_scale / l;
    uint16_t* row = p.out + out_row0 + (int64_t)h * D;
#pragma unroll
    for (int nb = 0; nb < Geo<KV, D>::NB; ++nb) {
      if constexpr (KV == 0) {  // 4 consecutive dims: one 8-byte store
        u32x2_t w = {f32_to_bf16_bits(st.acc[nb][0] * inv) | (f32_to_bf16_bits(st.acc[nb][1] * inv) << 16),
                     f32_to_bf16_bits(st.acc[nb][2] * inv) | (f32_to_bf16_bits(st.acc[nb][3] * inv) << 16)};
        *reinterpret_cast<u32x2_t*>(row + acc_dim<KV, D>(nb, 0, lane)) = w;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) store_bf16(row + acc_dim<KV, D>(nb, r, lane), st.acc[nb][r] * inv);
      }
    }
  }
}

template <int KV, int D>
__device__ __forceinline__ void wave_publish(MfmaState<KV, D>& st, const DecodeParams& p, int64_t slot, int lane) {
  float l = xor_sum(st.l, 16);
  l = xor_sum(l, 32);
  const int h = lane & 15;
  const int G = p.group;
  if (h < G) {
    float* acc = p.part_acc + (slot * G + h) * D;
#pragma unroll
    for (int nb = 0; nb < Geo<KV, D>::NB; ++nb) {
      if constexpr (KV == 0) {  // rows r = 0..3 are 4 consecutive dims
        *reinterpret_cast<f32x4_t*>(acc + acc_dim<KV, D>(nb, 0, lane)) = st.acc[nb];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[acc_dim<KV, D>(nb, r, lane)] = st.acc[nb][r];
      }
    }
    if (lane < 16) *reinterpret_cast<f32x2_t*>(p.part_ml + (slot * G + h) * 2) = f32x2_t{st.m, l};
  }
}

// A partial piece whose page ids failed the range check publishes m = +inf
// for every head (no valid partial has it); the merge then writes no output
// for the segment and adds the abort bit.
__device__ __forceinline__ void wave_publish_abort(const DecodeParams& p, int64_t slot, int lane) {
  for (int h = lane; h < p.group; h += 64)
    *reinterpret_cast<f32x2_t*>(p.part_ml + (slot * p.group + h) * 2) = f32x2_t{__builtin_huge_valf(), 0.f};
}

// VALU family: merge the 8 token slots (lanes differing in bits 3..5) first.
template <int KV, int D, int GM>
__device__ __forceinline__ void valu_merge_slots(ValuState<KV, D, GM>& st) {
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    float M = xor_max(st.m[h], 8);
    M = xor_max(M, 16);
    M = xor_max(M, 32);
    const float w = st.m[h] == kNegInf ? 0.f : fast_exp2(st.m[h] - M);
    float l = st.l[h] * w;
    l = xor_sum(l, 8);
    l = xor_sum(l, 16);
    st.l[h] = xor_sum(l, 32);
    st.m[h] = M;
#pragma unroll
    for (int i = 0; i < Geo<KV, D>::DC; ++i) {
      float a = st.acc[h][i] * w;
      a = xor_sum(a, 8);
      a = xor_sum(a, 16);
      st.acc[h][i] = xor_sum(a, 32);
    }
  }
}

template <int KV, int D, int GM>
__device__ __forceinline__ void wave_output(ValuState<KV, D, GM>& st, const DecodeParams& p, int64_t out_row0,
                                            int lane) {
  constexpr int DC = Geo<KV, D>::DC;
  valu_merge_slots(st);
  if (lane < 8) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < p.group) {
        const float inv = p.v_scale / st.l[h];
        uint16_t* row = p.out + out_row0 + (int64_t)h * D + lane * DC;
#pragma unroll
        for (int i = 0; i < DC; i += 2)
          *reinterpret_cast<uint32_t*>(row + i) =
              f32_to_bf16_bits(st.acc[h][i] * inv) | (f32_to_bf16_bits(st.acc[h][i + 1] * inv) << 16);
      }
    }
  }
}

template <int KV, int D, int GM>
__device__ __forceinline__ void wave_publish(ValuState<KV, D, GM>& st, const DecodeParams& p, int64_t slot,
                                             int lane) {
  constexpr int DC = Geo<KV, D>::DC;
  valu_merge_slots(st);
  const int G = p.group;
  if (lane < 8) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        float* acc = p.part_acc + (slot * G + h) * D + lane * DC;
#pragma unroll
        for (int i = 0; i < DC; i += 4)
          *reinterpret_cast<f32x4_t*>(acc + i) = f32x4_t{st.acc[h][i], st.acc[h][i + 1], st.acc[h][i + 2],
                                                         st.acc[h][i + 3]};
        if (lane == 0) *reinterpret_cast<f32x2_t*>(p.part_ml + (slot * G + h) * 2) = f32x2_t{st.m[h], st.l[h]};
      }
    }
  }
}

// ------------------------------------------------------------------------
// The balanced schedule.
//
// All work of one call is the flattened list of (sequence b, KV head g,
// tile t) triples, ordered b-major, then g, then t; sequence b contributes
// num_kv_heads segments of T_b = ceil(L_b / 64) tiles (0 for a sequence
// whose length is invalid).  Each segment occupies delta + T_b consecutive
// units of a flattened index: delta (0 or kPieceUnits) units that stand for
// the cost of starting a piece of it, then one unit per tile.  Wave w of
// the W = min(4 * num_blocks, TU) waves takes the contiguous unit range
// [w*TU/W, (w+1)*TU/W), so every wave gets the same work (+-1 unit) --
// tiles plus piece starts -- whatever the length mix: measured on MI355X, a
// wave's piece start (the query rows, the page ids and the first tile's
// loads, one after another) costs about 1.6 tile times, and with a charge of
// one unit the wave that starts 10 pieces over short sequences at batch 64
// ended ~15 us after the median wave.
// Each wave derives the schedule itself from seq_lens; the host never reads
// device memory, and waves never wait for one another.
//
// A wave's range is cut into pieces, one per segment whose tiles it holds
// (a range may end inside a segment's start charge).  A piece
// that is a whole segment is finished in registers.  Otherwise only the
// first and the last piece of a wave can be partial: the first is published
// in the wave's partial slot 0 (it starts at the range start), the last in
// slot 1.  A second kernel (one block per segment) merges the partials of
// waves wave_of(first tile) .. wave_of(last tile); the kernel boundary makes
// the partials visible to it, so no wave ever synchronizes with another.
// ------------------------------------------------------------------------
constexpr int64_t kSeqCount = int64_t(1) << 44;  // pass 1 packs a sequence count above the tile count
// A segment descriptor with this bit: a page id of the segment failed the
// decode's range check (tags off); nothing was written for it.
constexpr uint64_t kDescAbortMeta = uint64_t(1) << 63;
constexpr int kPieceUnits = 2;                    // schedule units a segment charges at its start
constexpr int64_t kMinTilesForCharge = 16;        // tiles per wave from which the charge applies
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t total, int64_t nw) { return w * total / nw; }
// the wave whose range holds flattened unit x
__device__ __forceinline__ int64_t wave_of(int64_t x, int64_t total, int64_t nw) { return ((x + 1) * nw - 1) / total; }

// tiles of sequence b's segments, 0 if it failed the page check
__device__ __forceinline__ int seq_tiles(int L, int max_tokens, uint32_t abort_bits) {
  return (abort_bits == 0 && L >= 1 && L <= max_tokens) ? (L + kTileTokens - 1) / kTileTokens : 0;
}

// Wave scans through DPP (register-to-register lane moves, no LDS round
// trips): row_shr:1,2,4,8 give inclusive prefix sums inside each row of 16
// lanes, row_bcast:15 and row_bcast:31 then carry the row totals into the
// rows above.  Lanes the pattern gives no source add the identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int64_t dpp_add64(int64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)((uint64_t)v >> 32), CTRL, ROW_MASK, 0xF, false);
  return v + (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ int64_t wave_inclusive_scan64(int64_t v) {
  v = dpp_add64<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add64<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add64<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add64<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add64<0x142, 0xA>(v);  // row_bcast:15 -> rows 1, 3
  v = dpp_add64<0x143, 0xC>(v);  // row_bcast:31 -> rows 2, 3
  return v;
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int i) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, i);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), i);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// One piece: tiles [t_lo, t_hi) of segment (b, g), whose flattened range is
// [seg_lo, seg_lo + T).
template <int KV, int D, int GM, bool MFMA>
__device__ __forceinline__ void wave_piece(const DecodeParams& p, uint8_t* vstage, int b, int g, int L, int T, int t_lo,
                                           int t_hi, int64_t seg_lo, int64_t r0, int64_t w, int64_t TT, int64_t nw,
                                           int lane) {
  const int G = p.group;
  typename WaveState<KV, D, GM, MFMA>::T st;
  const uint16_t* qrow0 = p.q + ((int64_t)b * p.num_q_heads + (int64_t)g * G) * D;
  if constexpr (MFMA) {
    using G_ = Geo<KV, D>;
    const int col = lane & 15;
    const int quarter = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < G_::KSTEPS; ++kk) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (col < G) v = *reinterpret_cast<const u32x4_t*>(qrow0 + (int64_t)col * D + quarter * (D / 4) + 8 * kk);
      st.q[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int nb_ = 0; nb_ < G_::NB; ++nb_) st.acc[nb_] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  } else {
    constexpr int DC = Geo<KV, D>::DC;
    const int dc = lane & 7;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      uint32_t v[DC / 2];
      if (h < G) {
        load_words<DC / 2>(reinterpret_cast<const uint8_t*>(qrow0 + (int64_t)h * D + dc * DC), v);
      } else {
#pragma unroll
        for (int i = 0; i < DC / 2; ++i) v[i] = 0u;
      }
#pragma unroll
      for (int i = 0; i < DC / 2; ++i) st.q2[h][i] = v[i];
      st.m[h] = kNegInf;
      st.l[h] = 0.f;
#pragma unroll
      for (int i = 0; i < DC; ++i) st.acc[h][i] = 0.f;
    }
  }

  const bool ok = run_wave<KV, D, GM, MFMA>(p, b, g, L, t_lo, t_hi - t_lo, st, lane, vstage);
  const int64_t seg = (int64_t)b * p.num_kv_heads + g;
  if (t_lo == 0 && t_hi == T) {
    // The whole segment is here: finish it (or, if one of its page ids was
    // out of range, write nothing and tell the merge kernel to flag it).
    if (lane == 0) p.seg_desc[seg] = ok ? 0 : kDescAbortMeta;
    if (ok) wave_output(st, p, ((int64_t)b * p.num_q_heads + (int64_t)g * G) * D, lane);
    return;
  }
  if (t_lo == 0 && lane == 0) {
    // The wave holding the segment's first tile tells the merge kernel
    // where the segment's partials are: first slot, number of partials.
    const uint32_t first_slot = (uint32_t)(2 * w + (r0 < seg_lo ? 1 : 0));
    const uint32_t n_part = (uint32_t)(wave_of(seg_lo + T - 1, TT, nw) - w + 1);
    p.seg_desc[seg] = first_slot | ((uint64_t)n_part << 32);
  }
  // A partial piece: publish it; the merge kernel combines the partials.
  const int64_t slot = 2 * w + ((seg_lo + t_lo) == r0 ? 0 : 1);
  if (ok)
    wave_publish(st, p, slot, lane);
  else
    wave_publish_abort(p, slot, lane);
}

// ------------------------------------------------------------------------
// The page check of a call with tags on (see page_check.hpp).
// ------------------------------------------------------------------------
__global__ __launch_bounds__(kBlockThreads) void check_kernel(DecodeParams p) {
  check_block(p, blockIdx.x, blockIdx.y);
}

// Abort bits of sequence b known before the decode: the OR of its chunks'
// check results when the page check ran, plus the length check.
__device__ __forceinline__ uint32_t seq_abort_bits(const DecodeParams& p, int b, int L, int max_tokens) {
  uint32_t bits = (L < 1 || L > max_tokens) ? kAbortMeta : 0u;
  if (p.checked)
    for (int c = 0; c < p.check_chunks; ++c) bits |= p.check_bits[(int64_t)b * p.check_chunks + c];
  return bits;
}

// ------------------------------------------------------------------------
// The kernel: 4 independent waves per block, each with an equal share.
// ------------------------------------------------------------------------
template <int KV, int D, int GM, bool MFMA>
__global__ __launch_bounds__(kBlockThreads, 1) void decode_kernel(DecodeParams p) {
  // FP8 MFMA family: one 64-token V tile per wave staged in LDS
  constexpr int kStage = (MFMA && KV == 0) ? kTileTokens * D : 16;
  __shared__ __attribute__((aligned(16))) uint8_t vstage_all[kWavesPerBlock][kStage];
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  uint8_t* vstage = vstage_all[threadIdx.x >> 6];
  const int max_tokens = p.max_pages << p.log2_page_size;
  const int64_t hkv = p.num_kv_heads;

  // ---- pass 1: total work of the sequences that passed the page check;
  // wave 0 writes every abort flag and marks the failed sequences' segments
  // as having nothing to merge
  // per lane: tiles (bits 0..43) + sequences with work (bits 44..) -- one scan for both
  int64_t mine = 0;
  int L0 = 0, T0 = 0;  // length and tiles of sequence `lane` (the first chunk of pass 2)
  for (int b = lane; b < p.batch; b += 64) {
    const int Lb = p.seq_lens[b];
    const uint32_t bits = seq_abort_bits(p, b, Lb, max_tokens);
    const int T = seq_tiles(Lb, max_tokens, bits);
    if (b == lane) {
      L0 = Lb;
      T0 = T;
    }
    mine += T + (T > 0 ? kSeqCount : 0);
    if (w == 0) {
      p.abort_flags[b] = (uint8_t)bits;
      if (T == 0)
        for (int g = 0; g < p.num_kv_heads; ++g) p.seg_desc[(int64_t)b * p.num_kv_heads + g] = 0;
    }
  }
  const int64_t packed = readlane64(wave_inclusive_scan64(mine), 63);
  const int64_t TT = (packed & (kSeqCount - 1)) * hkv;  // tiles of the whole call
  const int64_t n_segs = (packed / kSeqCount) * hkv;     // segments with work
  // Units: every segment charges kPieceUnits at its start on top of its
  // tiles, so a wave whose share starts pieces of several segments gets
  // fewer tiles (a piece's start costs about one tile time).  Only when the
  // shares are long enough for it to matter, so small calls keep one tile
  // per unit.
  const int64_t max_waves = (int64_t)p.num_blocks * kWavesPerBlock;
  const int delta = TT >= kMinTilesForCharge * max_waves ? kPieceUnits : 0;
  const int64_t TU = TT + delta * n_segs;
  // Never more shares than units (with delta > 0 a share is >= 16 units):
  // every wave inside a segment's span then holds some of its tiles.
  const int64_t nw = min(max_waves, TU);
  if (w >= nw) return;
  const int64_t r0 = range_start(w, TU, nw), r1 = range_start(w + 1, TU, nw);

  // ---- pass 2: walk the sequences 64 at a time, process the pieces in [r0, r1)
  int64_t carry = 0;  // units per KV head of all sequences before this chunk
  for (int c = 0; c < p.batch; c += 64) {
    if (carry * hkv >= r1) break;
    const int b = c + lane;
    // the first 64 sequences were read in pass 1: no second trip to memory
    const int Lc = c == 0 ? L0 : (b < p.batch ? p.seq_lens[b] : 0);
    const int T = c == 0 ? T0 : (b < p.batch ? seq_tiles(Lc, max_tokens, seq_abort_bits(p, b, Lc, max_tokens)) : 0);
    const int U = T > 0 ? T + delta : 0;  // units per KV head of sequence b
    const int64_t incl = wave_inclusive_scan64(U);
    const int64_t excl = carry + incl - U;
    const bool hit = U > 0 && excl * hkv < r1 && (excl + U) * hkv > r0;
    uint64_t mask = __ballot(hit);
    while (mask) {
      const int i = __builtin_ctzll(mask);
      mask &= mask - 1;
      const int Ti = __builtin_amdgcn_readlane(T, i);
      const int Ui = Ti + delta;
      const int bi = c + i;
      const int64_t seq_lo = readlane64(excl, i) * hkv;
      const int L = __builtin_amdgcn_readlane(Lc, i);
      const int64_t g_first = r0 > seq_lo ? (r0 - seq_lo) / Ui : 0;
      const int64_t g_last = min(hkv - 1, (r1 - 1 - seq_lo) / Ui);
      for (int64_t g = g_first; g <= g_last; ++g) {
        const int64_t seg_lo = seq_lo + g * Ui + delta;  // unit of the segment's first tile
        const int64_t lo = max(seg_lo, r0), hi = min(seg_lo + Ti, r1);
        if (lo >= hi) continue;  // this share holds only the segment's start charge
        wave_piece<KV, D, GM, MFMA>(p, vstage, bi, (int)g, L, Ti, (int)(lo - seg_lo), (int)(hi - seg_lo), seg_lo, r0,
                                    w, TU, nw, lane);
      }
    }
    carry += readlane64(incl, 63);
  }
}

// ------------------------------------------------------------------------
// The merge kernel: one item per (sequence, KV head, query head of the
// group), handled by WPI waves (1: four items per block; kWideMergeWaves:
// one item per block).  Segments
// finished inside one wave were written by the decode kernel, and aborted
// sequences have no descriptor; the others' partials are combined by
// log-sum-exp: M = max m_a, L = sum l_a 2^(m_a - M),
// o = v_scale * sum acc_a 2^(m_a - M) / L, rounded to BF16.  A segment with
// a piece that failed the decode's page-id range check (descriptor bit 63,
// or a partial with m = +inf) gets no output, and the item of its sequence's
// first KV head and first query head adds kAbortMeta to the abort flag (the
// decode kernel wrote the flag's other bits; every KV head's pieces read the
// same pages, so each segment reaches the same verdict).  The item's
// waves split its partials; lanes hold the statistics of up to 64 partials
// at a time and the head's output dims; each partial's accumulator row is
// one coalesced load per wave, kMergeUnroll of them in flight per lane; with
// WPI > 1 the waves' sums meet in LDS.  The host picks the wide form when
// the grid splits segments into many partials (small batches, long
// contexts).
// ------------------------------------------------------------------------
constexpr int kMergeUnroll = 16;
// Waves per query head when segments have many partials: at one 32k-token
// sequence (128 partials per segment) 8 waves of 16 partials each took
// 27.0 us per call, 4 waves of 32 27.6 us, 16 waves of 8 28.3 us.
constexpr int kWideMergeWaves = 8;

template <int D, int WPI>
__global__ __launch_bounds__(64 * (WPI > kWavesPerBlock ? WPI : kWavesPerBlock)) void merge_kernel(DecodeParams p) {
  constexpr int DL = D / 64;                                        // output dims per lane
  constexpr int WPB = WPI > kWavesPerBlock ? WPI : kWavesPerBlock;  // waves per block
  __shared__ float part_x[WPB][D];
  __shared__ float part_l[WPB];
  __shared__ float part_m[WPB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = wave % WPI, w0 = wave - sub;  // this wave's share of the item; the item's first wave
  const int G = p.group;
  const int64_t item = (int64_t)blockIdx.x * (WPB / WPI) + wave / WPI;
  if (item >= (int64_t)p.batch * p.num_q_heads) return;  // uniform over the item's waves
  const int64_t seg = item / G;
  const int h = (int)(item - seg * G);
  const int b = (int)(seg / p.num_kv_heads), g = (int)(seg - (int64_t)b * p.num_kv_heads);
  const uint64_t desc = p.seg_desc[seg];
  const bool flag_writer = g == 0 && h == 0 && sub == 0 && lane == 0;
  if (desc & kDescAbortMeta) {  // a whole segment that failed the range check
    if (flag_writer) p.abort_flags[b] |= (uint8_t)kAbortMeta;
    return;
  }
  const int n_arr = (int)(desc >> 32);
  if (n_arr < 2) return;  // finished inside one wave, or aborted by the page check
  const int64_t first_slot = (uint32_t)desc;
  const int64_t first = first_slot >> 1;
  // a descriptor always names slots of this call's waves; never read past them
  if (2 * (first + n_arr) > 2 * (int64_t)p.num_blocks * kWavesPerBlock) return;
  auto slot_of = [&](int a) -> int64_t { return a == 0 ? first_slot : 2 * (first + a); };
  // this wave's partials: [a_lo, a_hi)
  const int a_lo = (int)((int64_t)n_arr * sub / WPI);
  const int a_hi = (int)((int64_t)n_arr * (sub + 1) / WPI);

  // the maximum (lane j: partials a_lo + j, + 64, ...)
  float M = kNegInf, m0 = kNegInf, l0 = 0.f;
  for (int a = a_lo + lane; a < a_hi; a += 64) {
    const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(p.part_ml + (slot_of(a) * G + h) * 2);
    if (a < a_lo + 64) {
      m0 = ml[0];
      l0 = ml[1];
    }
    M = __builtin_fmaxf(M, ml[0]);
  }
  M = wave_max(M);
  if constexpr (WPI > 1) {
    if (lane == 0) part_m[wave] = M;
    __syncthreads();
    M = kNegInf;
#pragma unroll
    for (int i = 0; i < WPI; ++i) M = __builtin_fmaxf(M, part_m[w0 + i]);
  }
  if (M == __builtin_huge_valf()) {  // a piece failed the range check (uniform over the item's waves)
    if (flag_writer) p.abort_flags[b] |= (uint8_t)kAbortMeta;
    return;
  }

  // 64 partials at a time: lane j's weight 2^(m - M) is read by every lane
  float Ls = 0.f;
  float x[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) x[k] = 0.f;
  const float* acc_h = p.part_acc + (int64_t)h * D + lane * DL;
  for (int a0 = a_lo; a0 < a_hi; a0 += 64) {
    float m = m0, l = l0;
    if (a0 > a_lo && a0 + lane < a_hi) {
      const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(p.part_ml + (slot_of(a0 + lane) * G + h) * 2);
      m = ml[0];
      l = ml[1];
    }
    const float wgt = (a0 + lane < a_hi) ? fast_exp2(m - M) : 0.f;
    Ls += l * wgt;
    const int na = min(64, a_hi - a0);
    for (int j0 = 0; j0 < na; j0 += kMergeUnroll) {
      float v[kMergeUnroll][DL];
#pragma unroll
      for (int j = 0; j < kMergeUnroll; ++j) {
        const int jj = min(j0 + j, na - 1);  // past the end: re-read the last row, weight 0
        const float* src = acc_h + slot_of(a0 + jj) * G * D;
        if constexpr (DL == 2) {
          const f32x2_t t = *reinterpret_cast<const f32x2_t*>(src);
          v[j][0] = t[0];
          v[j][1] = t[1];
        } else {
          v[j][0] = *src;
        }
      }
#pragma unroll
      for (int j = 0; j < kMergeUnroll; ++j) {
        const int src_lane = min(j0 + j, 63);
        const float wj = j0 + j < na ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                    __builtin_bit_cast(int, wgt), src_lane))
                                     : 0.f;
#pragma unroll
        for (int k = 0; k < DL; ++k) x[k] += v[j][k] * wj;
      }
    }
  }
  Ls = wave_sum(Ls);
  if constexpr (WPI > 1) {
#pragma unroll
    for (int k = 0; k < DL; ++k) part_x[wave][lane * DL + k] = x[k];
    if (lane == 0) part_l[wave] = Ls;
    __syncthreads();
    if (sub != 0) return;
    Ls = 0.f;
#pragma unroll
    for (int k = 0; k < DL; ++k) x[k] = 0.f;
#pragma unroll
    for (int i = 0; i < WPI; ++i) {
      Ls += part_l[w0 + i];
#pragma unroll
      for (int k = 0; k < DL; ++k) x[k] += part_x[w0 + i][lane * DL + k];
    }
  }
  const float inv = p.v_scale / Ls;
  float o[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) o[k] = x[k] * inv;
  uint16_t* out = p.out + ((int64_t)b * p.num_q_heads + (int64_t)g * G + h) * D + lane * DL;
  if constexpr (DL == 2) {
    *reinterpret_cast<uint32_t*>(out) = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
  } else {
    *out = (uint16_t)f32_to_bf16_bits(o[0]);
  }
}

template <int KV, int D, int GM, bool MFMA>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (ev0 != nullptr) {
    const hipError_t e = hipEventRecord(ev0, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_kernel<KV, D, GM, MFMA>), dim3(p.num_blocks), dim3(kBlockThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1 != nullptr) {
    const hipError_t e1 = hipEventRecord(ev1, stream);
    if (e1 != hipSuccess) return e1;
  }
  const int64_t merge_items = (int64_t)p.batch * p.num_q_heads;  // one per query head
  // Segments split into many partials (more waves than 16 per segment when
  // every segment is as long as the page table allows) get kWideMergeWaves
  // waves per query head.
  const bool wide = (int64_t)p.num_blocks * kWavesPerBlock > 16 * (int64_t)p.batch * p.num_kv_heads;
  if (wide) {
    hipLaunchKernelGGL((merge_kernel<D, kWideMergeWaves>), dim3((unsigned)merge_items), dim3(64 * kWideMergeWaves), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((merge_kernel<D, 1>), dim3((unsigned)((merge_items + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(kBlockThreads), 0, stream, p);
  }
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_dtype_dim(const DecodeParams& p, bool mfma, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (mfma) return launch_one<KV, D, 16, true>(p, stream, ev0, ev1);
  if (p.group <= 1) return launch_one<KV, D, 1, false>(p, stream, ev0, ev1);
  if (p.group <= 2) return launch_one<KV, D, 2, false>(p, stream, ev0, ev1);
  return launch_one<KV, D, 4, false>(p, stream, ev0, ev1);
}

}  // namespace

hipError_t launch_page_check(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_kernel, dim3(p.check_chunks, p.batch), dim3(kBlockThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int kv_dtype, int head_dim, bool mfma, hipStream_t stream,
                         hipEvent_t decode_begin, hipEvent_t decode_end) {
  if (kv_dtype == 0) {
    if (head_dim == 64) return launch_dtype_dim<0, 64>(p, mfma, stream, decode_begin, decode_end);
    return launch_dtype_dim<0, 128>(p, mfma, stream, decode_begin, decode_end);
  }
  if (head_dim == 64) return launch_dtype_dim<1, 64>(p, mfma, stream, decode_begin, decode_end);
  return launch_dtype_dim<1, 128>(p, mfma, stream, decode_begin, decode_end);
}

}  // namespace fp8kv
