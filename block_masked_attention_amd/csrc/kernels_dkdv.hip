// gfx950 (CDNA4) key-tile backward kernel of block-diffusion attention: dK
// and dV of the clean K/V buffer and of the local corrupted keys, each summed
// over every local query that sees the key ("Block Parallelism for Efficient
// Distributed Long-Context Diffusion Language Model Training", §4.3, Backward
// pass; visibility of §3.2 in bdattn_mask.h). Operand layouts and the LDS tile
// format are described in device.h. This file is compiled on its own so that
// its scheduling options apply to this kernel only.
#include <stdlib.h>
#include <string.h>

#include "device.h"

namespace bdattn {
namespace {

using namespace dev;

// ======================================================================
// Backward, dK/dV. One workgroup = 8 waves owning BWD_TK keys of one KV head.
// Waves w and w + 4 (which share a SIMD) own the same 32 keys, in two roles:
//   the P wave    S = Q K^T, P = exp2(S c - LSE2) (masked), dV += P^T dO;
//   the dS wave   dP - D = dO V^T - D, dS = P (dP - D), dK += dS^T Q,
// with P handed over through LDS in the exact register layout in which both
// waves hold their 32 x 32 result tiles. Each step (BWD_TQ query rows of one
// q head) has two phases separated by a barrier: {S, P | dP} then {dV | dS,
// dK}, so in each phase one wave's vector work overlaps the other's matrix
// products. Each wave keeps one accumulator (dV or dK) and one operand (K or
// V) in registers, which lets two waves share a SIMD. The next step's Q and dO
// tiles and its LSE2 / -D values are copied into the other LDS buffer while the
// current one is in use. Tiles whose rows all see every key of the workgroup
// come first and skip the mask.
// ======================================================================
template <bool BF16, int D, int PREC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdArgs a) {
  // bdattn_precision: float32 dK, dV (>= 1); P and dS as two bf16 terms (2)
  constexpr bool OF32 = PREC >= 1, SPLIT = BF16 && PREC == 2;
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  constexpr int TK = BWD_TK, TQ = BWD_TQ, NW = 8, NMB = TQ / 32;
  constexpr int TSZ = TQ * D;
  static_assert(TK == 32 * NW / 2, "two waves per 32 keys");
  static_assert(TQ % 32 == 0 && TQ <= 128, "row data copy: one wave, 16 bytes per lane");
  __shared__ __attribute__((aligned(16))) T smem[4 * TSZ];        // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float r_row[2][2][TQ];  // [buffer][LSE2, -D]
  __shared__ __attribute__((aligned(16))) float4 p_hand[NW / 2][NMB][4][64];  // P handoff
  static_assert(sizeof(smem) + sizeof(r_row) + sizeof(p_hand) <= 160 * 1024, "LDS");
  constexpr uint32_t TB = TSZ * sizeof(T);  // bytes per tile

  const int wi = claim_item(a.claim_kv, a.n_kv_items);
  if (wi < 0) return;  // every item taken (the whole workgroup)
  const BwdItem item = a.kv_items[wi];
  const int it_x0 = item.x0, it_x1 = item.x1, it_c0 = item.c0, it_c1 = item.c1;
  const int it_xf = item.xf, it_cf = item.cf, it_xfe = item.xfe, it_cfe = item.cfe;
  const int kstream = item.hs & 1, kvh = item.hs >> 1;
  const int G = a.H / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3;            // key group: keys 32 kg .. 32 kg + 31 of the tile
  const bool p_role = wave < NW / 2;  // P wave (dV) or dS wave (dK)
  const int lk = lane & 31, hf = lane >> 5;
  const int key0 = item.ktile * TK;
  const int n_keys = kstream ? a.n_corr : a.n_clean_kv;
  const int my_key = key0 + 32 * kg + lk;
  const bool key_ok = my_key < n_keys;
  // Local query rows that see this lane's key form one interval per query
  // stream (§3.2 rules with row-nondecreasing bounds): [lo_c, hi_c) of the
  // clean rows and [lo_x, hi_x) of the corrupted rows.
  //   clean key at position p of block kb:  clean rows of blocks >= kb
  //     (token-causal: clean rows at positions >= p); corrupted rows of
  //     blocks with id > kb, i.e. from the first local block whose id exceeds
  //     kb. The item gives that block j0 for the tile's first key block k0/B;
  //     ids do not decrease, so a scan from j0 over the local blocks with ids
  //     in (k0/B, kb] finds it (a few blocks: the tile spans BWD_TK keys,
  //     and a repeated id is another copy of the same block);
  //   corrupted key of local block kb: the corrupted rows of that block (its
  //     own copy only);
  //   packed documents: no row after the end of the key's document.
  int lo_c = 0, hi_c = 0, lo_x = 0, hi_x = 0;
  if (key_ok) {
    // clean: global position and block (buffer row 0 is position
    // clean_kv_start); corrupted: local key and local block
    const int key_pos = kstream ? my_key : my_key + a.clean_kv_start;
    const int key_blk = key_pos / a.B;
    if (kstream) {
      lo_x = key_blk * a.B;
      hi_x = lo_x + a.B;
    } else {
      lo_c = max(0, (a.token_causal ? key_pos : key_blk * a.B) - a.clean_q_start);
      hi_c = a.n_clean_q;
      const int n_blk = a.n_corr / a.B;
      int j = it_x0 / a.B;  // j0: first local corrupted block with id > the tile's first block
      while (j < n_blk && a.ids[j] <= key_blk) ++j;
      lo_x = j * a.B;
      hi_x = a.n_corr;
      if (a.docs) {
        const BdDocSpan sp = a.docs[key_blk];
        hi_c = (int)min((int64_t)a.n_clean_q, max((int64_t)0, (int64_t)sp.hi - a.clean_q_start));
        hi_x = sp.xhi;
      }
    }
  }

  // a gathered clean buffer: this wave's 32 keys (inside one FWD_TK-key tile
  // of position order) sit at buffer rows key + kv_off
  int kv_off = 0;
  if (!kstream && a.kv_map && key0 + 32 * kg < n_keys) {
    const int g0 = key0 + 32 * kg;
    kv_off = a.kv_map[g0 / FWD_TK] * FWD_TK + g0 % FWD_TK - g0;
  }
  // this lane's key (P wave) or value (dS wave) as B operand, natural over d
  Frag kvf[D / 16];
  {
    const T* src = (const T*)(p_role ? (kstream ? a.k_x : a.k_c) : (kstream ? a.v_x : a.v_c));
    const int64_t off = ((int64_t)min(my_key, n_keys - 1) * a.Hkv + kvh) * D + (int64_t)kv_off * a.Hkv * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      kvf[ks] = key_ok ? E::load(src + off + 16 * ks + 8 * hf) : E::zero();
  }

  OperandReads<BF16, D> rd;
  rd.init(lane);

  f32x16 acc[D / 32];  // dV (P wave) or dK / scale (dS wave)
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = zero16();

  // Step order: the query tiles that see every key of the workgroup (those
  // inside [xf, xfe) / [cf, cfe)) come first, then the ones that need the
  // mask; within each, corrupted tiles then clean ones, each from the last
  // tile down, every q head of the group per tile. The masked tiles of a
  // stream are the u (0 or 1) tiles above the unmasked ones, then the tiles
  // below them. A step is (tile index t in that order, head offset hi),
  // advanced without divisions.
  auto ntiles = [](int r0, int r1) { return r1 > r0 ? (r1 - 1) / TQ - r0 / TQ + 1 : 0; };
  const int top_x = (it_x1 - 1) / TQ, top_c = (it_c1 - 1) / TQ;
  const int nf_x = ntiles(it_xf, it_xfe), nf_c = ntiles(it_cf, it_cfe);
  const int u_x = nf_x ? top_x - (it_xfe - 1) / TQ : 0;
  const int u_c = nf_c ? top_c - (it_cfe - 1) / TQ : 0;
  const int nm_x = ntiles(it_x0, it_x1) - nf_x, nm_c = ntiles(it_c0, it_c1) - nf_c;
  const int n_full = (nf_x + nf_c) * G;
  const int n_it = n_full + (nm_x + nm_c) * G;
  struct Step {
    int qs, q0, h;
  };
  struct Pos {
    int t, hi;
  };
  auto decode = [&](Pos p) __attribute__((always_inline)) {
    Step s;
    s.h = kvh * G + p.hi;
    int t = p.t;
    if (t < nf_x) {
      s.qs = 1;
      s.q0 = (top_x - u_x - t) * TQ;
    } else if ((t -= nf_x) < nf_c) {
      s.qs = 0;
      s.q0 = (top_c - u_c - t) * TQ;
    } else if ((t -= nf_c) < nm_x) {
      s.qs = 1;
      s.q0 = (top_x - (t < u_x ? 0 : nf_x) - t) * TQ;
    } else {
      t -= nm_x;
      s.qs = 0;
      s.q0 = (top_c - (t < u_c ? 0 : nf_c) - t) * TQ;
    }
    return s;
  };
  auto next_pos = [&](Pos p) __attribute__((always_inline)) {
    if (++p.hi == G) {
      p.hi = 0;
      ++p.t;
    }
    return p;
  };

  // per-lane source of the row-data copy: lanes [0, TQ/4) copy LSE2, the
  // next TQ/4 lanes -D (kept opaque so the per-step stream choice stays a
  // register select rather than a load of the selected argument)
  const float* rsrc_c = lane < TQ / 4 ? a.l2_c : a.d_c;
  const float* rsrc_x = lane < TQ / 4 ? a.l2_x : a.d_x;
  asm volatile("" : "+v"(rsrc_c), "+v"(rsrc_x));
  TileCopy<T, TQ, D, NW> cp;
  cp.init(wave, lane, (int64_t)a.H * D);
  // copy step s's Q and dO tiles and its LSE2 / -D rows into LDS buffer `buf`
  auto fetch = [&](const Step& s, int buf) __attribute__((always_inline)) {
    const int n_rows = s.qs ? a.n_corr : a.n_clean_q;
    const T* qsrc = (const T*)(s.qs ? a.q_x : a.q_c) + (int64_t)s.h * D;
    const T* gsrc = (const T*)(s.qs ? a.do_x : a.do_c) + (int64_t)s.h * D;
    T* dst = smem + buf * 2 * TSZ;
    cp.issue(dst, qsrc, s.q0, n_rows);
    cp.issue(dst + TSZ, gsrc, s.q0, n_rows);
    if (wave == 0 && lane < TQ / 2) {  // lanes [0, TQ/4): LSE2 of the TQ rows, then -D
      constexpr int L = TQ / 4;
      const int64_t r0 = (int64_t)s.h * row_pad(n_rows) + s.q0 + 4 * (lane % L);
      const float* src = (s.qs ? rsrc_x : rsrc_c) + r0;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(&r_row[buf][0][0])));
    }
  };

  // c += S (P wave) or dP (dS wave) of both row blocks of tile TILE against
  // this wave's keys / values, alternating blocks: product k = (ks, mb)
  auto scores = [&](auto tile_tag, f32x16* c) __attribute__((always_inline)) {
    constexpr uint32_t TILE = decltype(tile_tag)::value;
    product_chain<NMB * D / 16, kReadAhead, Frag>(
        [&](int k) __attribute__((always_inline)) { return rd.template row_frag<TILE>(smem, k % NMB, k / NMB); },
        [&](int k, const Frag& f) __attribute__((always_inline)) { E::mma(c[k % NMB], f, kvf[k / NMB]); });
  };
  // acc += X^T Y over the TQ rows of tile TILE, X given as packed result-order
  // fragments [block][half], Y the rows read transposed: product k = (16-row
  // slice mt, column block db)
  // (SPLIT: xl holds the remainders of x, a second product per fragment)
  auto accumulate = [&](auto tile_tag, const Frag (*x)[2], const Frag (*xl)[2]) __attribute__((always_inline)) {
    constexpr uint32_t TILE = decltype(tile_tag)::value;
    product_chain<NMB * 2 * (D / 32), kReadAhead, Frag>(
        [&](int k) __attribute__((always_inline)) {
          return rd.template tr_frag<TILE>(smem, 16 * (k / (D / 32)), k % (D / 32));
        },
        [&](int k, const Frag& y) __attribute__((always_inline)) {
          const int mt = k / (D / 32);
          E::mma(acc[k % (D / 32)], x[mt / 2][mt % 2], y);
          if constexpr (SPLIT) E::mma(acc[k % (D / 32)], xl[mt / 2][mt % 2], y);
        });
  };

  Pos pos = {0, 0};  // position of the current step
  // P wave: S, P (masked on tiles that need it), hand P over, dV += P^T dO
  auto body_p = [&](auto mask_tag, auto buf_tag, int i) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;
    using QT = std::integral_constant<uint32_t, BUF * 2 * TB>;
    using GT = std::integral_constant<uint32_t, BUF * 2 * TB + TB>;
    const Pos nxt = next_pos(pos);
    if (i + 1 < n_it) fetch(decode(nxt), BUF ^ 1);
    const Step st = decode(pos);
    const int n_rows = st.qs ? a.n_corr : a.n_clean_q;
    // visibility of (query row, this lane's key) on tiles that need the mask
    const int lo = st.qs ? lo_x : lo_c, hi = st.qs ? hi_x : hi_c;
    auto sees = [&](int row) __attribute__((always_inline)) { return row >= lo && row < hi; };
    f32x16 sb[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) sb[mb] = zero16();
    // S first: the raised priority gives the S chain the matrix core, so P's
    // exponentials then overlap the dS wave's dP products
    __builtin_amdgcn_s_setprio(2);
    scores(QT{}, sb);
    __builtin_amdgcn_s_setprio(0);
    Frag pa[NMB][2], pl[NMB][2];  // P (and its remainder when SPLIT)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const f32x16& s = sb[mb];
      float p[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr = 32 * mb + 8 * g + 4 * hf;
        const float4 l4 = *(const float4*)(&r_row[BUF][0][qr]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pv = fast_exp2(fmaf(s[4 * g + r], a.scale_log2, -lv[r]));
          if (MASK) pv = sees(st.q0 + qr + r) ? pv : 0.f;
          p[4 * g + r] = pv;
        }
        p_hand[kg][mb][g][lane] = make_float4(p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]);
      }
      if constexpr (SPLIT) {
        split_pack(p, pa[mb][0], pl[mb][0]);
        split_pack(p + 8, pa[mb][1], pl[mb][1]);
      } else {
        pa[mb][0] = E::pack(p);
        pa[mb][1] = E::pack(p + 8);
      }
    }
    __syncthreads();  // P handed over
    accumulate(GT{}, pa, pl);
    pos = nxt;
    lds_dma_wait();
    __syncthreads();
  };
  // dS wave: dP - D (the product accumulates onto -D, read from LDS in the
  // result layout: element i of a row block is row 8(i/4) + 4 h + i%4), then
  // (once P is there) dS = P (dP - D), dK += dS^T Q
  auto body_ds = [&](auto buf_tag, int i) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    using QT = std::integral_constant<uint32_t, BUF * 2 * TB>;
    using GT = std::integral_constant<uint32_t, BUF * 2 * TB + TB>;
    const Pos nxt = next_pos(pos);
    if (i + 1 < n_it) fetch(decode(nxt), BUF ^ 1);
    f32x16 dp[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = *(const float4*)(&r_row[BUF][1][32 * mb + 8 * g + 4 * hf]);
        dp[mb][4 * g + 0] = d4.x;
        dp[mb][4 * g + 1] = d4.y;
        dp[mb][4 * g + 2] = d4.z;
        dp[mb][4 * g + 3] = d4.w;
      }
    }
    scores(GT{}, dp);
    __syncthreads();  // P handed over
    // dS ahead of the P wave's dV products, so that the dK products start early
    __builtin_amdgcn_s_setprio(2);
    Frag sa[NMB][2], sl[NMB][2];  // dS (and its remainder when SPLIT)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      float ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 p4 = p_hand[kg][mb][g][lane];
        ds[4 * g + 0] = p4.x * dp[mb][4 * g + 0];
        ds[4 * g + 1] = p4.y * dp[mb][4 * g + 1];
        ds[4 * g + 2] = p4.z * dp[mb][4 * g + 2];
        ds[4 * g + 3] = p4.w * dp[mb][4 * g + 3];
      }
      if constexpr (SPLIT) {
        split_pack(ds, sa[mb][0], sl[mb][0]);
        split_pack(ds + 8, sa[mb][1], sl[mb][1]);
      } else {
        sa[mb][0] = E::pack(ds);
        sa[mb][1] = E::pack(ds + 8);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    accumulate(QT{}, sa, sl);
    pos = nxt;
    lds_dma_wait();
    __syncthreads();
  };
  auto sweep_p = [&](auto mask_tag, int i0, int i1) __attribute__((always_inline)) {
    int i = i0;
    if (i < i1 && (i & 1)) body_p(mask_tag, Int<1>{}, i++);
    for (; i + 1 < i1; i += 2) {
      body_p(mask_tag, Int<0>{}, i);
      body_p(mask_tag, Int<1>{}, i + 1);
    }
    if (i < i1) body_p(mask_tag, Int<0>{}, i);
  };

  if (n_it > 0) fetch(decode(pos), 0);
  vm_drain();
  __syncthreads();
  if (p_role) {
    sweep_p(std::false_type{}, 0, n_full);
    sweep_p(std::true_type{}, n_full, n_it);
  } else {
    int i = 0;
    for (; i + 1 < n_it; i += 2) {
      body_ds(Int<0>{}, i);
      body_ds(Int<1>{}, i + 1);
    }
    if (i < n_it) body_ds(Int<0>{}, i);
  }

  // write dV (P wave) or dK times the scale (dS wave) for this pair's 32 keys
  void* out = p_role ? (kstream ? a.dv_x : a.dv_c) : (kstream ? a.dk_x : a.dk_c);
  const float osc = p_role ? 1.f : a.scale;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + 32 * kg + 8 * (i >> 2) + 4 * hf + (i & 3);
      const int64_t o = ((int64_t)(key + kv_off) * a.Hkv + kvh) * D + 32 * db + lk;
      if (key < n_keys) {
        if constexpr (OF32) ((float*)out)[o] = acc[db][i] * osc;
        else ((T*)out)[o] = E::from_f(acc[db][i] * osc);
      }
    }
  }
}

}  // namespace

hipError_t launch_dkdv(const BwdArgs& a, int dtype, int d, hipStream_t s) {
  if (a.n_kv_items <= 0) return hipSuccess;
  if (const char* e = getenv("BDATTN_DKDV"); e && !strcmp(e, "fused") && !a.precision)
    return launch_dkdv_fused(a, dtype, d, s);
  const dim3 grid(a.n_kv_items + (a.claim_kv ? claim_extra(a.n_kv_items) : 0)), block(512);
  const int pr = dtype == BDATTN_BF16 ? a.precision : 0;  // bdattn_precision (bf16 inputs)
  if (dtype == BDATTN_BF16 && d == 128 && pr == 2) hipLaunchKernelGGL((bwd_dkdv_kernel<true, 128, 2>), grid, block, 0, s, a);
  else if (dtype == BDATTN_BF16 && d == 128 && pr == 1) hipLaunchKernelGGL((bwd_dkdv_kernel<true, 128, 1>), grid, block, 0, s, a);
  else if (dtype == BDATTN_BF16 && d == 128) hipLaunchKernelGGL((bwd_dkdv_kernel<true, 128, 0>), grid, block, 0, s, a);
  else if (dtype == BDATTN_BF16 && d == 32 && pr == 2) hipLaunchKernelGGL((bwd_dkdv_kernel<true, 32, 2>), grid, block, 0, s, a);
  else if (dtype == BDATTN_BF16 && d == 32 && pr == 1) hipLaunchKernelGGL((bwd_dkdv_kernel<true, 32, 1>), grid, block, 0, s, a);
  else if (dtype == BDATTN_BF16 && d == 32) hipLaunchKernelGGL((bwd_dkdv_kernel<true, 32, 0>), grid, block, 0, s, a);
  else if (dtype == BDATTN_F32 && d == 32) hipLaunchKernelGGL((bwd_dkdv_kernel<false, 32, 0>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bdattn
