// gfx950 (CDNA4) kernels of block-diffusion attention: forward, backward
// preprocessing and the backward's dQ kernel, plus the launches (the key-tile
// dK/dV kernel lives in kernels_dkdv.hip).
//
// Forward and backward of the attention described in "Block Parallelism for
// Efficient Distributed Long-Context Diffusion Language Model Training":
// §3.2 gives the visibility (bdattn_mask.h); the appendix's "Efficient fused
// operator" paragraph gives the shape of the operator: the forward covers the
// clean-K/V part and the block-diagonal corrupted part and saves O and the
// log-sum-exp; the backward reuses them and returns dQ, the local corrupted
// dK/dV and the clean dK/dV summed over every local query that sees each
// clean key (§4.3, Backward pass).
//
// Kernels:
//   fwd_kernel       query-tile parallel: online softmax over the visible keys
//   bwd_prep_kernel  -D = -rowsum(dO * O) and LSE * log2(e) per query row
//   bwd_dq_kernel    query-tile parallel: dQ = scale * dS K, written once
//   bwd_dkdv_kernel  key-tile parallel: dV = P^T dO, dK = scale * dS^T Q over
//                    every query tile (and q head of the KV group) that sees
//                    the keys, written once (kernels_dkdv.hip)
//   merge_kernel     two partial results over disjoint key sets -> one
// No output is accumulated with atomics (the only atomics are the work-claim
// counters, claim_item in device.h), so every output is bitwise reproducible.
//
// Matrix products use the CDNA4 32x32x16 bf16 MFMA (fp32 accumulate), or, for
// fp32 problems, eight 32x32x2 fp32 MFMAs per 16-deep step. The softmax is the
// online normaliser (Milakov & Gimelshein, cited by the pages) in fp32, in
// base 2 with the scale folded into one multiply. Operand layouts and the LDS
// tile format are described in device.h.
//
// Tile loops are double buffered with the buffer index a compile-time
// constant of the loop body (two copies of each body), so every LDS operand
// read carries its buffer in the instruction's immediate offset.
#include <stdlib.h>
#include <string.h>

#include "device.h"

namespace bdattn {

// dQ launches for problems with packed documents. They live in a translation
// unit of their own (kernels_dq_docs.hip, which compiles this file's kernels
// with BDATTN_DQ_DOCS_UNIT defined) so that they can be built with another
// machine scheduler than the rest of this file: the register-minimising
// schedule that suits the other query-tile kernels makes this variant spill.
template <bool BF16, int D, int PREC, bool MAPPED, bool PERSIST>
void launch_dq_docs(const BwdArgs& a, dim3 grid, dim3 block, hipStream_t s);

namespace {

using namespace dev;

// ======================================================================
// Query-tile work item shared by the forward and the dQ kernel: `rows`
// consecutive rows of one stream for Gw q heads of one KV group; wave w covers
// 32 rows of one head. The keys are swept in tiles of TK staged through LDS
// (K and V, row-major, double buffered): the clean keys [first clo, last cb),
// then, for corrupted rows, the local corrupted keys of their blocks. Clean
// tiles [jf0, jf1) lie inside every row's clean interval and skip the mask;
// without packed documents (DOCS false) every clo is 0 and j0 = jf0 = 0.
// ======================================================================
struct QTile {
  int stream, head, kvh, n_rows, row0, my_row, crow, n_ct, n_xt, xlo, j0, jf0, jf1;
  bool row_ok;
  BdRowBounds rb;
};

template <int TK, bool DOCS>
__device__ __forceinline__ QTile q_tile(const FwdItem& it, int rows_per_item, int Gw, int H,
                                        int Hkv, int n_clean_q, int n_corr, const RowSpace& rs,
                                        int wave, int lq) {
  QTile q;
  q.stream = it.hs & 1;
  const int hg = it.hs >> 1;
  q.head = hg * Gw + (wave % Gw);
  q.kvh = q.head / (H / Hkv);
  q.n_rows = q.stream ? n_corr : n_clean_q;
  q.row0 = it.tile * rows_per_item;
  const int row_end = min(q.n_rows, q.row0 + rows_per_item);
  q.my_row = q.row0 + (wave / Gw) * 32 + lq;
  q.row_ok = q.my_row < q.n_rows;
  q.crow = min(q.my_row, q.n_rows - 1);
  BdRowBounds b[3];  // this lane's row, the item's first and last rows
  row_bounds3(q.stream, {q.crow, q.row0, row_end - 1}, rs, b);
  q.rb = b[0];
  const BdRowBounds first = b[1], last = b[2];
  q.j0 = DOCS ? first.clo / TK : 0;
  // (with documents, rows that see no clean key at all sweep none)
  q.n_ct = DOCS && last.cb <= first.clo ? q.j0 : (last.cb + TK - 1) / TK;
  q.jf0 = DOCS ? min(q.n_ct, max(q.j0, (last.clo + TK - 1) / TK)) : 0;
  q.jf1 = max(q.jf0, min(q.n_ct, first.cb / TK));
  q.xlo = q.stream ? first.xlo : 0;
  q.n_xt = q.stream ? (last.xhi - first.xlo + TK - 1) / TK : 0;
  return q;
}

// ======================================================================
// Forward. Per key tile: S^T = K Q^T (keys x queries, so each lane owns one
// query row); mask only on tiles that need it; online softmax; O^T += V^T P^T.
// ======================================================================
template <bool BF16, int D, bool DOCS, bool MAPPED, int PREC, bool PERSIST = false>
__global__ __launch_bounds__(FWD_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdArgs a) {
  // bdattn_precision: float32 O (>= 1); P as two bf16 terms in P V (2)
  constexpr bool OF32 = PREC >= 1, SPLIT = BF16 && PREC == 2;
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  constexpr int TK = FWD_TK;
  constexpr int TSZ = TK * D;
  static_assert(4 * TSZ * sizeof(T) <= 80 * 1024, "LDS (two workgroups per CU)");
  __shared__ __attribute__((aligned(16))) T smem[4 * TSZ];  // [buffer][K, V]
  constexpr uint32_t TB = TSZ * sizeof(T);                   // bytes per tile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const RowSpace rs{a.clean_q_start, a.B, a.ids, a.token_causal != 0, a.clean_kv_start,
                    a.n_clean_kv, a.corr_keys != 0, DOCS ? a.docs : nullptr};
  // The workgroup's items: the one claim_item gives it, or, when PERSIST, one
  // claim after another until every queue is empty (a short work list on a
  // grid of one workgroup per CU: each next item starts while the previous
  // one's stores are in flight, with no workgroup launch in between; on long
  // lists it is claimed during the previous item's start, beside its loads).
  // (claimed ahead only on long lists: with few items per workgroup, a late
  // claim balances the end of the list better)
  const bool ahead = PERSIST && a.n_items >= 16 * a.persist;
  for (int wi = claim_item(a.claim, a.n_items), next = -1; wi >= 0 && wi < a.n_items; wi = next) {
    const QTile q = q_tile<TK, DOCS>(a.items[wi], a.rows_per_item, a.Gw, a.H, a.Hkv,
                               a.n_clean_q, a.n_corr, rs, wave, lq);
    const int n_tiles = q.n_ct + q.n_xt;
    const T* qsrc = (const T*)(q.stream ? a.q_x : a.q_c);

    // Q as the B operand of S^T = K Q^T: column = this lane's row, natural over d
    Frag qf[D / 16];
    {
      const T* qrow = qsrc + ((int64_t)q.crow * a.H + q.head) * D;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = q.row_ok ? E::load(qrow + 16 * ks + 8 * hf) : E::zero();
    }

    // the first CW waves copy the key tiles. A tile's copies pass the CU's
    // memory pipeline at about 64 bytes a cycle, and a wave waits at each of
    // its copies until the pipeline takes it; the older wave of each SIMD,
    // which runs ahead of its partner, absorbs that wait, and the younger one
    // starts its products at once.
    constexpr int CW = FWD_COPY_WAVES;
    TileCopy<T, TK, D, CW> cp;
    cp.init(wave, lane, (int64_t)a.Hkv * D);
    const T* const kc = (const T*)a.k_c + (int64_t)q.kvh * D;
    const T* const kx = (const T*)a.k_x + (int64_t)q.kvh * D;
    const T* const vc = (const T*)a.v_c + (int64_t)q.kvh * D;
    const T* const vx = (const T*)a.v_x + (int64_t)q.kvh * D;
    // gathered buffer (MAPPED): clean key tile j (position order) sits at
    // buffer tile kv_map[j]; the masks keep working in position order
    KeyTileMap<TK> km;
    if constexpr (MAPPED) {
      if (q.n_ct > q.j0) km.init(a.kv_map, a.n_kv_map, q.j0, lane);
    }
    // stage key tile j (K then V) into LDS buffer `buf`
    auto fetch = [&](int j, int buf) __attribute__((always_inline)) {
      const bool cl = j < q.n_ct;
      int k0;
      if constexpr (MAPPED) k0 = cl ? km.row(j, lane) : q.xlo + (j - q.n_ct) * TK;
      else k0 = cl ? j * TK : q.xlo + (j - q.n_ct) * TK;
      const int nk = cl ? a.n_clean_kv : a.n_corr;
      T* dst = smem + buf * 2 * TSZ;
      if (CW == FWD_WAVES || wave < CW) {
        cp.issue(dst, cl ? kc : kx, k0, nk);
        cp.issue(dst + TSZ, cl ? vc : vx, k0, nk);
      }
    };

    OperandReads<BF16, D> rd;
    rd.init(lane);

    f32x16 o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] = zero16();
    float m = kNegInf, l = 0.f;  // running reference maximum (log2 units), row sum

    // one key tile in LDS buffer BUF (the next one is copied into the other)
    auto body = [&](auto mask_tag, auto buf_tag, int j) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      constexpr int BUF = decltype(buf_tag)::value;
      constexpr uint32_t KT = BUF * 2 * TB, VT = KT + TB;
      if (j + 1 < n_tiles) fetch(j + 1, BUF ^ 1);
      const bool cl = j < q.n_ct;
      const int k0 = cl ? j * TK : q.xlo + (j - q.n_ct) * TK;

      // S of both key blocks, alternating blocks: product k = (ks, mb)
      f32x16 s[TK / 32];
#pragma unroll
      for (int mb = 0; mb < TK / 32; ++mb) s[mb] = zero16();
      product_chain<TK / 32 * D / 16, kReadAhead, Frag>(
          [&](int k) __attribute__((always_inline)) { return rd.template row_frag<KT>(smem, k % (TK / 32), k / (TK / 32)); },
          [&](int k, const Frag& f) __attribute__((always_inline)) { E::mma(s[k % (TK / 32)], f, qf[k / (TK / 32)]); });
      // online softmax; the row max is taken on raw scores (the scale is > 0)
      // and the scale folded into the exponent's multiply-add
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < TK / 32; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (MASK) {
            const int key = k0 + 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3);
            // (documents: clo <= key < cb as one unsigned compare; a test of the
            // same form as the corrupted one lets the compiler pick the bound
            // fields by address, which moves the bounds to scratch memory)
            const bool vis = cl ? (DOCS ? uint32_t(key - q.rb.clo) < uint32_t(q.rb.cb - q.rb.clo)
                                        : key < q.rb.cb)
                                : bd_sees_corr(q.rb, key);
            s[mb][i] = vis ? s[mb][i] : kNegInf;
          }
          mx = fmaxf(mx, s[mb][i]);
        }
      }
      mx = max_halves(mx) * a.scale_log2;
      if (__any(mx > m + kRescaleMargin)) {  // some row's maximum moved (wave-uniform)
        const float m_new = fmaxf(m, mx);
        const float alpha = m == kNegInf ? 0.f : fast_exp2(m - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }
        m = m_new;
      }
      const float m_use = m == kNegInf ? 0.f : m;
      // the row sum adds the fp32 weights: LSE must be exact, since the
      // backward rebuilds P from it (summing the bf16-rounded weights instead
      // shifts LSE by up to 2^-9 and scales every recomputed P of the row)
      Frag pf[TK / 32][2], pl[TK / 32][2];  // P (and its remainder when SPLIT)
      float rs = 0.f;
      // weights of the 16-key slice mt (8 per lane), elements [i0, i1); packed
      // to bf16 once complete
      float pv[8];
      auto weights = [&](int mt, int i0, int i1) __attribute__((always_inline)) {
        const int mb = mt / 2, h = mt % 2;
#pragma unroll
        for (int i = i0; i < i1; ++i) {
          pv[i] = fast_exp2(fmaf(s[mb][8 * h + i], a.scale_log2, -m_use));
          rs += pv[i];
        }
        if (i1 == 8) {
          if constexpr (SPLIT) split_pack(pv, pf[mb][h], pl[mb][h]);
          else pf[mb][h] = E::pack(pv);
        }
      };
      // O += V^T P over the tile's keys: product k = (16-key slice mt, column
      // block db). Slice 0's weights come first; slice mt + 1's are computed
      // between the products of slice mt (same values and summation order as
      // computing them all first).
      constexpr int PS = D / 32;   // products per slice
      constexpr int EPP = 8 / PS;  // weights computed after each product
      weights(0, 0, 8);
      product_chain_hooked<TK / 32 * 2 * PS, kReadAhead, Frag>(
          [&](int k) __attribute__((always_inline)) { return rd.template tr_frag<VT>(smem, 16 * (k / PS), k % PS); },
          [&](int k, const Frag& y) __attribute__((always_inline)) {
            const int mt = k / PS;
            E::mma(o[k % PS], y, pf[mt / 2][mt % 2]);
            if constexpr (SPLIT) E::mma(o[k % PS], y, pl[mt / 2][mt % 2]);
          },
          [&](int k) __attribute__((always_inline)) {
            const int mt = k / PS, db = k % PS;
            if (mt + 1 < TK / 16) weights(mt + 1, db * EPP, (db + 1) * EPP);
          });
      l += rs;
      lds_dma_wait();
      __syncthreads();
    };
    auto sweep = [&](auto mask_tag, int j0, int j1) __attribute__((always_inline)) {
      int j = j0;
      if (j < j1 && (j & 1)) body(mask_tag, Int<1>{}, j++);
      for (; j + 1 < j1; j += 2) {
        body(mask_tag, Int<0>{}, j);
        body(mask_tag, Int<1>{}, j + 1);
      }
      if (j < j1) body(mask_tag, Int<0>{}, j);
    };
    if (n_tiles > q.j0) fetch(q.j0, q.j0 & 1);
    if constexpr (PERSIST) {
      if (ahead) next = claim_item(a.claim, a.n_items);
    }
    vm_drain();
    __syncthreads();
    // tiles [jf0, jf1) lie inside every row's clean interval and skip the mask
    if constexpr (DOCS) sweep(std::true_type{}, q.j0, q.jf0);
    sweep(std::false_type{}, q.jf0, q.jf1);
    sweep(std::true_type{}, q.jf1, n_tiles);

    const float lt = l + __shfl_xor(l, 32);
    if (q.row_ok) {
      // a row that sees no key present (partial problems): O = 0, LSE = -inf
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int64_t orow = ((int64_t)q.my_row * a.H + q.head) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store_out<E, OF32>(q.stream ? a.o_x : a.o_c, orow + 32 * db + 8 * g + 4 * hf,
                             o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                             o[db][4 * g + 3] * inv);
      }
      if (hf == 0) {
        float* lse = q.stream ? a.lse_x : a.lse_c;
        lse[(int64_t)q.head * q.n_rows + q.my_row] = lt > 0.f ? (m + log2f(lt)) * kLn2 : kNegInf;
      }
    }
    if constexpr (PERSIST) {
      if (!ahead) next = claim_item(a.claim, a.n_items);
    }
  }
}

// ======================================================================
// Backward preprocess: per (row, head) -D = -rowsum(dO * O) and LSE * log2(e),
// D/8 lanes each, written [H][n_pad]; rows n..n_pad-1 get D = 0, LSE = +inf
// (query tiles past the end of a stream then contribute nothing). D is stored
// negated so that the dK/dV kernel can start its dP accumulation from it.
// ======================================================================
template <bool BF16, int D, bool OF32>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const void* o_, const void* do_,
                                                       const float* lse, float* Dout, float* L2out,
                                                       int32_t n_rows, int32_t n_pad, int32_t H) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int LPR = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = idx / LPR;
  const int sub = int(idx % LPR);
  const int64_t npairs = (int64_t)n_pad * H;
  const int64_t row = pair / H, head = pair % H;
  const bool real = pair < npairs && row < n_rows;
  float acc = 0.f;
  if (real) {
    typename E::Frag fg = E::load((const T*)do_ + pair * D + 8 * sub);
    const T* pg = (const T*)&fg;
    if constexpr (OF32 && BF16) {  // float32 O
      const float4* po = (const float4*)((const float*)o_ + pair * D + 8 * sub);
      const float4 x = po[0], y = po[1];
      const float ov[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += ov[e] * E::to_f(pg[e]);
    } else {
      typename E::Frag fo = E::load((const T*)o_ + pair * D + 8 * sub);
      const T* po = (const T*)&fo;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += E::to_f(po[e]) * E::to_f(pg[e]);
    }
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, LPR);
  if (pair < npairs && sub == 0) {
    Dout[head * n_pad + row] = real ? -acc : 0.f;
    L2out[head * n_pad + row] = real ? lse[head * n_rows + row] * kLog2e : __builtin_inff();
  }
}

// ======================================================================
// Merge of two partial results over disjoint key sets (the appendix's
// Implementation 1): per (row, head) LSE = ln(exp LSE_a + exp LSE_b) and
// O = exp(LSE_a - LSE) O_a + exp(LSE_b - LSE) O_b; a part with LSE = -inf
// weighs 0, and a row with no key in either part gets O = 0, LSE = -inf.
// D/8 lanes per (row, head), all in one wave, so each lane reads its inputs
// before any lane writes (outputs may alias inputs).
// ======================================================================
template <bool BF16, int D>
__global__ __launch_bounds__(256) void merge_kernel(const void* oa_, const float* la,
                                                    const void* ob_, const float* lb, void* o_,
                                                    float* lse, int64_t n_rows, int32_t H) {
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  constexpr int LPR = D / 8;
  static_assert(64 % LPR == 0, "a (row, head) in one wave");
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = idx / LPR;  // row * H + head
  const int sub = int(idx % LPR);
  if (pair >= n_rows * H) return;
  const int64_t row = pair / H, head = pair % H;
  const int64_t li = head * n_rows + row;
  const float a = la[li], b = lb[li];
  const float m = fmaxf(a, b);
  float wa = 0.f, wb = 0.f, l = kNegInf;
  if (m != kNegInf) {
    wa = expf(a - m);  // exp(-inf) = 0
    wb = expf(b - m);
    const float den = wa + wb;
    l = m + logf(den);
    wa /= den;
    wb /= den;
  }
  const int64_t off = pair * D + 8 * sub;
  const Frag fa = E::load((const T*)oa_ + off), fb = E::load((const T*)ob_ + off);
  const T* ea = (const T*)&fa;
  const T* eb = (const T*)&fb;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = wa * E::to_f(ea[e]) + wb * E::to_f(eb[e]);
  *(Frag*)((T*)o_ + off) = E::pack(x);
  if (sub == 0) lse[li] = l;
}

// ======================================================================
// Backward, dQ. Same query tiles and key sweep as the forward. Per key tile:
// S^T = K Q^T and dP^T = V dO^T (each lane owns one query row, so its LSE and
// D are scalars); P^T = exp2(S^T c - LSE2); dS^T = P^T (dP^T - D);
// dQ^T += K^T dS^T with K^T read transposed from the K tile.
// ======================================================================
template <bool BF16, int D, bool DOCS, bool MAPPED, int PREC, bool PERSIST = false>
__global__ __launch_bounds__(FWD_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a) {
  // bdattn_precision: float32 dQ (>= 1); dS as two bf16 terms in dS K (2)
  constexpr bool OF32 = PREC >= 1, SPLIT = BF16 && PREC == 2;
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  constexpr int TK = FWD_TK;
  constexpr int TSZ = TK * D;
  static_assert(4 * TSZ * sizeof(T) <= 80 * 1024, "LDS (two workgroups per CU)");
  __shared__ __attribute__((aligned(16))) T smem[4 * TSZ];  // [buffer][K, V]
  constexpr uint32_t TB = TSZ * sizeof(T);                   // bytes per tile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const RowSpace rs{a.clean_q_start, a.B, a.ids, a.token_causal != 0, a.clean_kv_start,
                    a.n_clean_kv, a.corr_keys != 0, DOCS ? a.docs : nullptr};
  // The workgroup's items: the one claim_item gives it, or, when PERSIST, one
  // claim after another until every queue is empty (a short work list on a
  // grid of one workgroup per CU: each next item starts while the previous
  // one's stores are in flight, with no workgroup launch in between; on long
  // lists it is claimed during the previous item's start, beside its loads).
  // (claimed ahead only on long lists: with few items per workgroup, a late
  // claim balances the end of the list better)
  const bool ahead = PERSIST && a.n_q_items >= 16 * a.persist;
  for (int wi = claim_item(a.claim_q, a.n_q_items), next = -1; wi >= 0 && wi < a.n_q_items; wi = next) {
    const QTile q = q_tile<TK, DOCS>(a.q_items[wi], a.rows_per_item, a.Gw, a.H, a.Hkv,
                               a.n_clean_q, a.n_corr, rs, wave, lq);
    const int n_tiles = q.n_ct + q.n_xt;
    const T* qsrc = (const T*)(q.stream ? a.q_x : a.q_c);
    const T* gsrc = (const T*)(q.stream ? a.do_x : a.do_c);

    Frag qf[D / 16], gf[D / 16];
    {
      const int64_t off = ((int64_t)q.crow * a.H + q.head) * D;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        qf[ks] = q.row_ok ? E::load(qsrc + off + 16 * ks + 8 * hf) : E::zero();
        gf[ks] = q.row_ok ? E::load(gsrc + off + 16 * ks + 8 * hf) : E::zero();
      }
    }
    const int64_t ri = (int64_t)q.head * row_pad(q.n_rows) + q.crow;
    const float lse2 = q.row_ok ? (q.stream ? a.l2_x : a.l2_c)[ri] : __builtin_inff();
    const float ndrow = q.row_ok ? (q.stream ? a.d_x : a.d_c)[ri] : 0.f;  // -D

    TileCopy<T, TK, D, FWD_WAVES> cp;
    cp.init(wave, lane, (int64_t)a.Hkv * D);
    const T* const kc = (const T*)a.k_c + (int64_t)q.kvh * D;
    const T* const kx = (const T*)a.k_x + (int64_t)q.kvh * D;
    const T* const vc = (const T*)a.v_c + (int64_t)q.kvh * D;
    const T* const vx = (const T*)a.v_x + (int64_t)q.kvh * D;
    // gathered buffer (MAPPED): clean key tile j (position order) sits at
    // buffer tile kv_map[j]; the masks keep working in position order
    KeyTileMap<TK> km;
    if constexpr (MAPPED) {
      if (q.n_ct > q.j0) km.init(a.kv_map, a.n_kv_map, q.j0, lane);
    }
    // stage key tile j (K then V) into LDS buffer `buf`
    auto fetch = [&](int j, int buf) __attribute__((always_inline)) {
      const bool cl = j < q.n_ct;
      int k0;
      if constexpr (MAPPED) k0 = cl ? km.row(j, lane) : q.xlo + (j - q.n_ct) * TK;
      else k0 = cl ? j * TK : q.xlo + (j - q.n_ct) * TK;
      const int nk = cl ? a.n_clean_kv : a.n_corr;
      T* dst = smem + buf * 2 * TSZ;
      cp.issue(dst, cl ? kc : kx, k0, nk);
      cp.issue(dst + TSZ, cl ? vc : vx, k0, nk);
    };

    OperandReads<BF16, D> rd;
    rd.init(lane);

    f32x16 dq[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dq[i] = zero16();

    auto body = [&](auto mask_tag, auto buf_tag, int j) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      constexpr int BUF = decltype(buf_tag)::value;
      constexpr uint32_t KT = BUF * 2 * TB, VT = KT + TB;
      if (j + 1 < n_tiles) fetch(j + 1, BUF ^ 1);
      const bool cl = j < q.n_ct;
      const int k0 = cl ? j * TK : q.xlo + (j - q.n_ct) * TK;
      Frag sf[TK / 32][2], sl[TK / 32][2];  // dS (and its remainder when SPLIT)
#pragma unroll
      for (int mb = 0; mb < TK / 32; ++mb) {
        // S and dP of key block mb, alternating: even k S (K rows), odd k dP (V rows)
        f32x16 s = zero16(), dp = zero16();
        product_chain<2 * D / 16, kReadAhead, Frag>(
            [&](int k) __attribute__((always_inline)) {
              return (k & 1) ? rd.template row_frag<VT>(smem, mb, k / 2) : rd.template row_frag<KT>(smem, mb, k / 2);
            },
            [&](int k, const Frag& f) __attribute__((always_inline)) {
              if (k & 1) E::mma(dp, f, gf[k / 2]);
              else E::mma(s, f, qf[k / 2]);
            });
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(fmaf(s[i], a.scale_log2, -lse2));
          if (MASK) {
            const int key = k0 + 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3);
            // (documents: clo <= key < cb as one unsigned compare; a test of the
            // same form as the corrupted one lets the compiler pick the bound
            // fields by address, which moves the bounds to scratch memory)
            const bool vis = cl ? (DOCS ? uint32_t(key - q.rb.clo) < uint32_t(q.rb.cb - q.rb.clo)
                                        : key < q.rb.cb)
                                : bd_sees_corr(q.rb, key);
            p = vis ? p : 0.f;
          }
          ds[i] = p * (dp[i] + ndrow);
        }
        if constexpr (SPLIT) {
          split_pack(ds, sf[mb][0], sl[mb][0]);
          split_pack(ds + 8, sf[mb][1], sl[mb][1]);
        } else {
          sf[mb][0] = E::pack(ds);
          sf[mb][1] = E::pack(ds + 8);
        }
      }
      // dQ += K^T dS over the tile's keys: product k = (16-key slice mt, column block db)
      product_chain<TK / 32 * 2 * (D / 32), kReadAhead, Frag>(
          [&](int k) __attribute__((always_inline)) { return rd.template tr_frag<KT>(smem, 16 * (k / (D / 32)), k % (D / 32)); },
          [&](int k, const Frag& y) __attribute__((always_inline)) {
            const int mt = k / (D / 32);
            E::mma(dq[k % (D / 32)], y, sf[mt / 2][mt % 2]);
            if constexpr (SPLIT) E::mma(dq[k % (D / 32)], y, sl[mt / 2][mt % 2]);
          });
      lds_dma_wait();
      __syncthreads();
    };
    auto sweep = [&](auto mask_tag, int j0, int j1) __attribute__((always_inline)) {
      int j = j0;
      if (j < j1 && (j & 1)) body(mask_tag, Int<1>{}, j++);
      for (; j + 1 < j1; j += 2) {
        body(mask_tag, Int<0>{}, j);
        body(mask_tag, Int<1>{}, j + 1);
      }
      if (j < j1) body(mask_tag, Int<0>{}, j);
    };
    if (n_tiles > q.j0) fetch(q.j0, q.j0 & 1);
    if constexpr (PERSIST) {
      if (ahead) next = claim_item(a.claim_q, a.n_q_items);
    }
    vm_drain();
    __syncthreads();
    // tiles [jf0, jf1) lie inside every row's clean interval and skip the mask
    if constexpr (DOCS) sweep(std::true_type{}, q.j0, q.jf0);
    sweep(std::false_type{}, q.jf0, q.jf1);
    sweep(std::true_type{}, q.jf1, n_tiles);

    if (q.row_ok) {
      const int64_t orow = ((int64_t)q.my_row * a.H + q.head) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store_out<E, OF32>(q.stream ? a.dq_x : a.dq_c, orow + 32 * db + 8 * g + 4 * hf,
                             dq[db][4 * g] * a.scale, dq[db][4 * g + 1] * a.scale,
                             dq[db][4 * g + 2] * a.scale, dq[db][4 * g + 3] * a.scale);
      }
    }
    if constexpr (PERSIST) {
      if (!ahead) next = claim_item(a.claim_q, a.n_q_items);
    }
  }
}

#ifndef BDATTN_DQ_DOCS_UNIT
template <bool BF16, int D, int PREC>
hipError_t run_fwd_t(const FwdArgs& a, hipStream_t s, const KernelEvents* ev) {
  if (ev) (void)hipEventRecord(ev[0].start, s);
  const dim3 grid(a.n_items + (a.claim ? claim_extra(a.n_items) : 0)), block(FWD_WAVES * 64);
  if constexpr (BF16 && D == 128 && PREC == 0) {
    if (a.n_items > 0 && a.persist > 0) {  // (the host sets persist only without kv_map)
      if (a.docs) hipLaunchKernelGGL((fwd_kernel<BF16, D, true, false, PREC, true>), dim3(a.persist), block, 0, s, a);
      else hipLaunchKernelGGL((fwd_kernel<BF16, D, false, false, PREC, true>), dim3(a.persist), block, 0, s, a);
      if (ev) (void)hipEventRecord(ev[0].stop, s);
      return hipGetLastError();
    }
  }
  if (a.n_items > 0 && a.kv_map) {  // a gathered clean buffer
    if (a.docs) hipLaunchKernelGGL((fwd_kernel<BF16, D, true, true, PREC>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<BF16, D, false, true, PREC>), grid, block, 0, s, a);
  } else if (a.n_items > 0) {
    if (a.docs) hipLaunchKernelGGL((fwd_kernel<BF16, D, true, false, PREC>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<BF16, D, false, false, PREC>), grid, block, 0, s, a);
  }
  if (ev) (void)hipEventRecord(ev[0].stop, s);
  return hipGetLastError();
}

// the precisions other than the default are separate instantiations for bf16
// inputs only (float32 inputs have float32 outputs and operands already)
template <bool BF16, int D>
hipError_t run_fwd(const FwdArgs& a, hipStream_t s, const KernelEvents* ev) {
  if constexpr (BF16) {
    if (a.precision == BDATTN_PRECISION_SPLIT) return run_fwd_t<BF16, D, 2>(a, s, ev);
    if (a.precision == BDATTN_PRECISION_F32_OUT) return run_fwd_t<BF16, D, 1>(a, s, ev);
  }
  return run_fwd_t<BF16, D, 0>(a, s, ev);
}

template <bool BF16, int D, int PREC>
hipError_t run_bwd_t(const BwdArgs& a, hipStream_t s, const KernelEvents* ev) {
  constexpr int LPR = D / 8;
  for (int st = 0; st < 2; ++st) {
    const int32_t n = st ? a.n_corr : a.n_clean_q;
    if (n == 0) continue;
    const int32_t n_pad = row_pad(n);
    const int64_t threads = (int64_t)n_pad * a.H * LPR;
    const int blocks = int((threads + 255) / 256);
    hipLaunchKernelGGL((bwd_prep_kernel<BF16, D, (PREC >= 1)>), dim3(blocks), dim3(256), 0, s,
                       st ? a.o_x : a.o_c, st ? a.do_x : a.do_c, st ? a.lse_x : a.lse_c,
                       st ? a.d_x : a.d_c, st ? a.l2_x : a.l2_c, n, n_pad, a.H);
  }
  // BDATTN_BWD=fused10: the one-kernel backward (timed in the dK/dV slot)
  const int dtype = BF16 ? BDATTN_BF16 : BDATTN_F32;
  if (const char* e = getenv("BDATTN_BWD"); e && !strcmp(e, "fused10") && bwd_fused_supported(a, dtype, D)) {
    if (ev) (void)hipEventRecord(ev[0].start, s);
    if (ev) (void)hipEventRecord(ev[0].stop, s);
    if (ev) (void)hipEventRecord(ev[1].start, s);
    const hipError_t err = launch_bwd_fused(a, dtype, D, s);
    if (ev) (void)hipEventRecord(ev[1].stop, s);
    return err;
  }
  if (ev) (void)hipEventRecord(ev[0].start, s);
  const dim3 grid(a.n_q_items + (a.claim_q ? claim_extra(a.n_q_items) : 0)), block(FWD_WAVES * 64);
  bool launched = false;
  if constexpr (BF16 && D == 128 && PREC == 0) {
    if (a.n_q_items > 0 && a.persist > 0) {  // (the host sets persist only without kv_map)
      if (a.docs) launch_dq_docs<BF16, D, PREC, false, true>(a, dim3(a.persist), block, s);
      else hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, false, false, PREC, true>), dim3(a.persist), block, 0, s, a);
      launched = true;
    }
  }
  if (launched || a.n_q_items <= 0) {
  } else if (a.kv_map) {  // a gathered clean buffer
    if (a.docs) launch_dq_docs<BF16, D, PREC, true, false>(a, grid, block, s);
    else hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, false, true, PREC>), grid, block, 0, s, a);
  } else {
    if (a.docs) launch_dq_docs<BF16, D, PREC, false, false>(a, grid, block, s);
    else hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, false, false, PREC>), grid, block, 0, s, a);
  }
  if (ev) (void)hipEventRecord(ev[0].stop, s);
  if (ev) (void)hipEventRecord(ev[1].start, s);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_dkdv(a, dtype, D, s);
  if (ev) (void)hipEventRecord(ev[1].stop, s);
  return e;
}

template <bool BF16, int D>
hipError_t run_bwd(const BwdArgs& a, hipStream_t s, const KernelEvents* ev) {
  if constexpr (BF16) {
    if (a.precision == BDATTN_PRECISION_SPLIT) return run_bwd_t<BF16, D, 2>(a, s, ev);
    if (a.precision == BDATTN_PRECISION_F32_OUT) return run_bwd_t<BF16, D, 1>(a, s, ev);
  }
  return run_bwd_t<BF16, D, 0>(a, s, ev);
}

}  // namespace

bool have_kernels(int dtype, int d) {
  if (dtype == BDATTN_BF16) return d == 32 || d == 128;
  if (dtype == BDATTN_F32) return d == 32;
  return false;
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int d, hipStream_t s, const KernelEvents* ev) {
  if (dtype == BDATTN_BF16 && d == 128) return run_fwd<true, 128>(a, s, ev);
  if (dtype == BDATTN_BF16 && d == 32) return run_fwd<true, 32>(a, s, ev);
  if (dtype == BDATTN_F32 && d == 32) return run_fwd<false, 32>(a, s, ev);
  return hipErrorInvalidValue;
}

template <bool BF16, int D>
hipError_t run_merge(int64_t n_rows, int H, const void* o_a, const float* lse_a, const void* o_b,
                     const float* lse_b, void* o, float* lse, hipStream_t s) {
  const int64_t threads = n_rows * H * (D / 8);
  if (threads > 0)
    hipLaunchKernelGGL((merge_kernel<BF16, D>), dim3(unsigned((threads + 255) / 256)), dim3(256), 0,
                       s, o_a, lse_a, o_b, lse_b, o, lse, n_rows, H);
  return hipGetLastError();
}

hipError_t launch_merge(int64_t n_rows, int H, int d, int dtype, const void* o_a,
                        const float* lse_a, const void* o_b, const float* lse_b, void* o,
                        float* lse, hipStream_t s) {
  if (dtype == BDATTN_BF16 && d == 128) return run_merge<true, 128>(n_rows, H, o_a, lse_a, o_b, lse_b, o, lse, s);
  if (dtype == BDATTN_BF16 && d == 32) return run_merge<true, 32>(n_rows, H, o_a, lse_a, o_b, lse_b, o, lse, s);
  if (dtype == BDATTN_F32 && d == 32) return run_merge<false, 32>(n_rows, H, o_a, lse_a, o_b, lse_b, o, lse, s);
  if (dtype == BDATTN_F32 && d == 128) return run_merge<false, 128>(n_rows, H, o_a, lse_a, o_b, lse_b, o, lse, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, int d, hipStream_t s, const KernelEvents* ev) {
  if (dtype == BDATTN_BF16 && d == 128) return run_bwd<true, 128>(a, s, ev);
  if (dtype == BDATTN_BF16 && d == 32) return run_bwd<true, 32>(a, s, ev);
  if (dtype == BDATTN_F32 && d == 32) return run_bwd<false, 32>(a, s, ev);
  return hipErrorInvalidValue;
}
#else  // BDATTN_DQ_DOCS_UNIT
}  // namespace

template <bool BF16, int D, int PREC, bool MAPPED, bool PERSIST>
void launch_dq_docs(const BwdArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, true, MAPPED, PREC, PERSIST>), grid, block, 0, s, a);
}

// the variants run_bwd_t launches: every (dtype, d, precision) with and
// without a gathered buffer, and the persistent grid of bf16, d = 128
#define BDATTN_DQ_DOCS(BF16, D, PREC)                                                         \
  template void launch_dq_docs<BF16, D, PREC, false, false>(const BwdArgs&, dim3, dim3, hipStream_t); \
  template void launch_dq_docs<BF16, D, PREC, true, false>(const BwdArgs&, dim3, dim3, hipStream_t);
BDATTN_DQ_DOCS(true, 128, 0)
BDATTN_DQ_DOCS(true, 128, 1)
BDATTN_DQ_DOCS(true, 128, 2)
BDATTN_DQ_DOCS(true, 32, 0)
BDATTN_DQ_DOCS(true, 32, 1)
BDATTN_DQ_DOCS(true, 32, 2)
BDATTN_DQ_DOCS(false, 32, 0)
#undef BDATTN_DQ_DOCS
template void launch_dq_docs<true, 128, 0, false, true>(const BwdArgs&, dim3, dim3, hipStream_t);
#endif  // BDATTN_DQ_DOCS_UNIT

}  // namespace bdattn
