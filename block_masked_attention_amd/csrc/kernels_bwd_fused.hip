// gfx950 (CDNA4) single-wave-per-SIMD backward kernels of block-diffusion
// attention ("Block Parallelism for Efficient Distributed Long-Context
// Diffusion Language Model Training", §4.3, Backward pass), kept as measured
// alternatives to the split backward (kernels.hip dQ + kernels_dkdv.hip):
//
//   dK/dV with fused roles (BDATTN_DKDV=fused): one wave per 32 keys does S,
//     P, dP, dS, dV and dK itself, the vector work placed between its own
//     matrix products, with no P hand-over and one barrier per step. Same
//     results bit for bit as the split dK/dV kernel; on MI355X 5-7% slower at
//     64K and 256K (a lone wave per SIMD leaves the matrix core idle while it
//     does vector work).
//   The whole backward in one kernel (BDATTN_BWD=fused10, bf16, d = 128,
//     contiguous clean K/V): the same kernel also forms dQ = c dS K from dS
//     (transposed through LDS) and the workgroup's keys, and adds it into a
//     float32 buffer with float atomics; a last pass rounds it into dQ. 10 d
//     flops per pair and q head instead of 14 d, but every step adds a
//     64 x 128 float32 tile into memory, and on this memory the atomics are
//     resolved beyond the L2 at about 1.2 TB/s, which bounds the kernel.
//
// Both run the split kernel's work list and step order.
#include <map>
#include <mutex>

#include "device.h"

namespace bdattn {
namespace {

using namespace dev;

// ======================================================================
// One workgroup = 4 waves (one per SIMD) owning BWD_TK keys of one KV head,
// 32 per wave. Each wave keeps K, V and both accumulators of its 32 keys in
// registers and runs, per step of BWD_TQ query rows of one q head, product
// chains on the step's Q and dO tiles:
//   S = Q K^T;
//   dP - D = dO V^T onto -D, with P = exp2(S c - LSE2) (masked) computed
//     between its products;
//   dV += P^T dO, with dS = P (dP - D) computed between its products;
//   dK += dS^T Q;
//   (DQ) dQ[:, 32 w .. 32 w + 31] += dS K over the workgroup's 128 keys, from
//     dS^T and K in LDS, then float atomic adds into dq_acc [rows][H][D] (clean
//     rows, then corrupted rows).
// ======================================================================
template <bool BF16, int D, bool DQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_fused_kernel(BwdArgs a, float* dq_acc) {
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  constexpr int TK = BWD_TK, TQ = BWD_TQ, NW = 4, NMB = TQ / 32;
  constexpr int TSZ = TQ * D;
  static_assert(TK == 32 * NW, "one wave per 32 keys");
  static_assert(TQ % 32 == 0 && TQ <= 128, "row data copy: one wave, 16 bytes per lane");
  __shared__ __attribute__((aligned(16))) T smem[4 * TSZ];        // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float r_row[2][2][TQ];  // [buffer][LSE2, -D]
  constexpr uint32_t TB = TSZ * sizeof(T);  // bytes per tile
  // with dQ: the workgroup's keys [TK][D] and dS transposed [TK keys][TQ rows]
  __shared__ __attribute__((aligned(16))) T k_lds[DQ ? TK * D : 8];
  __shared__ __attribute__((aligned(16))) T dst_lds[DQ ? TK * TQ : 8];
  static_assert(sizeof(smem) + sizeof(r_row) + sizeof(k_lds) + sizeof(dst_lds) <= 160 * 1024, "LDS");

  const BwdItem item = a.kv_items[blockIdx.x];
  const int it_x0 = item.x0, it_x1 = item.x1, it_c0 = item.c0, it_c1 = item.c1;
  const int it_xf = item.xf, it_cf = item.cf, it_xfe = item.xfe, it_cfe = item.cfe;
  const int kstream = item.hs & 1, kvh = item.hs >> 1;
  const int G = a.H / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lk = lane & 31, hf = lane >> 5;
  const int key0 = item.ktile * TK;
  const int n_keys = kstream ? a.n_corr : a.n_clean_kv;
  const int my_key = key0 + 32 * wave + lk;
  const bool key_ok = my_key < n_keys;
  // rows that see this lane's key: one interval per query stream (the rules
  // of the split dK/dV kernel)
  int lo_c = 0, hi_c = 0, lo_x = 0, hi_x = 0;
  if (key_ok) {
    const int key_pos = kstream ? my_key : my_key + a.clean_kv_start;
    const int key_blk = key_pos / a.B;
    if (kstream) {
      lo_x = key_blk * a.B;
      hi_x = lo_x + a.B;
    } else {
      lo_c = max(0, (a.token_causal ? key_pos : key_blk * a.B) - a.clean_q_start);
      hi_c = a.n_clean_q;
      const int n_blk = a.n_corr / a.B;
      int j = it_x0 / a.B;
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
  // a gathered clean buffer: this wave's 32 keys sit at buffer rows key + kv_off
  int kv_off = 0;
  if (!kstream && a.kv_map && key0 + 32 * wave < n_keys) {
    const int g0 = key0 + 32 * wave;
    kv_off = a.kv_map[g0 / FWD_TK] * FWD_TK + g0 % FWD_TK - g0;
  }
  // this lane's key and value as B operands, natural over d
  Frag kf[D / 16], vf[D / 16];
  {
    const T* ks = (const T*)(kstream ? a.k_x : a.k_c);
    const T* vs = (const T*)(kstream ? a.v_x : a.v_c);
    const int64_t off = ((int64_t)min(my_key, n_keys - 1) * a.Hkv + kvh) * D + (int64_t)kv_off * a.Hkv * D;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
      kf[k] = key_ok ? E::load(ks + off + 16 * k + 8 * hf) : E::zero();
      vf[k] = key_ok ? E::load(vs + off + 16 * k + 8 * hf) : E::zero();
    }
  }

  OperandReads<BF16, D> rd;
  rd.init(lane);
  OperandReads<BF16, TQ> rdt;  // the dS^T tile (TQ columns)
  if constexpr (DQ) {
    rdt.init(lane);
    TileCopy<T, TK, D, NW> kc;
    kc.init(wave, lane, (int64_t)a.Hkv * D);
    kc.issue(k_lds, (const T*)(kstream ? a.k_x : a.k_c) + (int64_t)kvh * D, key0, n_keys);
  }

  f32x16 acck[D / 32], accv[D / 32];  // dK / scale, dV
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acck[i] = accv[i] = zero16();

  // step order as in bwd_dkdv_kernel
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
  const float* rsrc_c = lane < TQ / 4 ? a.l2_c : a.d_c;
  const float* rsrc_x = lane < TQ / 4 ? a.l2_x : a.d_x;
  asm volatile("" : "+v"(rsrc_c), "+v"(rsrc_x));
  TileCopy<T, TQ, D, NW> cp;
  cp.init(wave, lane, (int64_t)a.H * D);
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
  // acc += X^T Y over the TQ rows of tile TILE, X packed result-order
  // fragments [block][half], Y the rows read transposed; hook(k) after product k
  auto accumulate = [&](auto tile_tag, f32x16* acc, const Frag (*x)[2], auto hook)
      __attribute__((always_inline)) {
    constexpr uint32_t TILE = decltype(tile_tag)::value;
    product_chain_hooked<NMB * 2 * (D / 32), kReadAhead, Frag>(
        [&](int k) __attribute__((always_inline)) {
          return rd.template tr_frag<TILE>(smem, 16 * (k / (D / 32)), k % (D / 32));
        },
        [&](int k, const Frag& y) __attribute__((always_inline)) {
          const int mt = k / (D / 32);
          E::mma(acc[k % (D / 32)], x[mt / 2][mt % 2], y);
        },
        hook);
  };

  constexpr int NP = NMB * D / 16;           // products of the S and dP chains
  constexpr int NE = NMB * 16;               // result elements per lane
  constexpr int EPS = NE / NP;               // elements handled after each S/dP product
  constexpr int EPA = NE / (NMB * 2 * (D / 32));  // ... after each dV product
  static_assert(NE % NP == 0 && NE % (NMB * 2 * (D / 32)) == 0, "elements per product");

  Pos pos = {0, 0};
  auto body = [&](auto mask_tag, auto buf_tag, int i) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;
    using QT = std::integral_constant<uint32_t, BUF * 2 * TB>;
    using GT = std::integral_constant<uint32_t, BUF * 2 * TB + TB>;
    const Pos nxt = next_pos(pos);
    if (i + 1 < n_it) fetch(decode(nxt), BUF ^ 1);
    const Step st = decode(pos);
    const int lo = st.qs ? lo_x : lo_c, hi = st.qs ? hi_x : hi_c;
    // this step's LSE2 and -D in the result layout: element i of row block
    // mb is row 32 mb + 8 (i/4) + 4 hf + i%4
    float l2[NMB][16];
    f32x16 dp[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr = 32 * mb + 8 * g + 4 * hf;
        const float4 l4 = *(const float4*)(&r_row[BUF][0][qr]);
        const float4 d4 = *(const float4*)(&r_row[BUF][1][qr]);
        l2[mb][4 * g] = l4.x, l2[mb][4 * g + 1] = l4.y, l2[mb][4 * g + 2] = l4.z, l2[mb][4 * g + 3] = l4.w;
        dp[mb][4 * g] = d4.x, dp[mb][4 * g + 1] = d4.y, dp[mb][4 * g + 2] = d4.z, dp[mb][4 * g + 3] = d4.w;
      }
    }
    // S = Q K^T of both row blocks, alternating blocks: product k = (ks, mb)
    f32x16 sb[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) sb[mb] = zero16();
    product_chain<NP, kReadAhead, Frag>(
        [&](int k) __attribute__((always_inline)) { return rd.template row_frag<QT::value>(smem, k % NMB, k / NMB); },
        [&](int k, const Frag& f) __attribute__((always_inline)) { E::mma(sb[k % NMB], f, kf[k / NMB]); });
    // dP - D = dO V^T onto -D; P between its products
    float pw[NMB][16];
    Frag pa[NMB][2];
    product_chain_hooked<NP, kReadAhead, Frag>(
        [&](int k) __attribute__((always_inline)) { return rd.template row_frag<GT::value>(smem, k % NMB, k / NMB); },
        [&](int k, const Frag& f) __attribute__((always_inline)) { E::mma(dp[k % NMB], f, vf[k / NMB]); },
        [&](int k) __attribute__((always_inline)) {
#pragma unroll
          for (int e = k * EPS; e < (k + 1) * EPS; ++e) {
            const int mb = e / 16, ii = e % 16;
            float pv = fast_exp2(fmaf(sb[mb][ii], a.scale_log2, -l2[mb][ii]));
            if (MASK) {
              const int row = st.q0 + 32 * mb + 8 * (ii >> 2) + 4 * hf + (ii & 3);
              pv = (row >= lo && row < hi) ? pv : 0.f;
            }
            pw[mb][ii] = pv;
            if (ii == 7) pa[mb][0] = E::pack(pw[mb]);
            if (ii == 15) pa[mb][1] = E::pack(pw[mb] + 8);
          }
        });
    // dV += P^T dO; dS = P (dP - D) between its products
    float dsw[NMB][16];
    Frag sa[NMB][2];
    accumulate(GT{}, accv, pa, [&](int k) __attribute__((always_inline)) {
#pragma unroll
      for (int e = k * EPA; e < (k + 1) * EPA; ++e) {
        const int mb = e / 16, ii = e % 16;
        // (keys past the end: zero, as their K rows feed dQ)
        dsw[mb][ii] = (!DQ || key_ok) ? pw[mb][ii] * dp[mb][ii] : 0.f;
        if (ii == 7) sa[mb][0] = E::pack(dsw[mb]);
        if (ii == 15) sa[mb][1] = E::pack(dsw[mb] + 8);
      }
    });
    if constexpr (DQ) {
      // dS^T into LDS: this lane's key is tile row 32 wave + lk; its values
      // of rows 32 mb + 8 g + 4 hf + (0..3) are 4 consecutive columns
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint4 v = sa[mb][g >> 1].v;
          const uint2 w2 = (g & 1) ? make_uint2(v.z, v.w) : make_uint2(v.x, v.y);
          *(uint2*)(dst_lds + tile_off<TQ, 8>(32 * wave + lk, 32 * mb + 8 * g + 4 * hf)) = w2;
        }
      }
    }
    // dK += dS^T Q
    accumulate(QT{}, acck, sa, [](int) {});
    if constexpr (DQ) {
      __syncthreads();  // dS^T of all keys written
      // dQ[:, 32 wave .. +32] += dS K over the workgroup's keys; result lane
      // l holds column 32 wave + l%32, element i row 32 mb + 8(i/4) + 4 hf + i%4
      f32x16 dq[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) dq[mb] = zero16();
#pragma unroll
      for (int ks = 0; ks < TK / 16; ++ks) {
        const Frag kb = rd.template tr_frag<0>(k_lds, 16 * ks, wave);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) E::mma(dq[mb], rdt.template tr_frag<0>(dst_lds, 16 * ks, mb), kb);
      }
      const int n_rows = st.qs ? a.n_corr : a.n_clean_q;
      float* acc = dq_acc + (st.qs ? (int64_t)a.n_clean_q * a.H * D : 0) + (int64_t)st.h * D + 32 * wave + lk;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = st.q0 + 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (row < n_rows) unsafeAtomicAdd(acc + (int64_t)row * a.H * D, dq[mb][i]);
        }
      }
    }
    pos = nxt;
    lds_dma_wait();
    __syncthreads();
  };
  auto sweep = [&](auto mask_tag, int i0, int i1) __attribute__((always_inline)) {
    int i = i0;
    if (i < i1 && (i & 1)) body(mask_tag, Int<1>{}, i++);
    for (; i + 1 < i1; i += 2) {
      body(mask_tag, Int<0>{}, i);
      body(mask_tag, Int<1>{}, i + 1);
    }
    if (i < i1) body(mask_tag, Int<0>{}, i);
  };

  if (n_it > 0) fetch(decode(pos), 0);
  vm_drain();
  __syncthreads();
  sweep(std::false_type{}, 0, n_full);
  sweep(std::true_type{}, n_full, n_it);

  T* outv = (T*)(kstream ? a.dv_x : a.dv_c);
  T* outk = (T*)(kstream ? a.dk_x : a.dk_c);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + 32 * wave + 8 * (i >> 2) + 4 * hf + (i & 3);
      if (key < n_keys) {
        const int64_t o = ((int64_t)(key + kv_off) * a.Hkv + kvh) * D + 32 * db + lk;
        outv[o] = E::from_f(accv[db][i]);
        outk[o] = E::from_f(acck[db][i] * a.scale);
      }
    }
  }
}

__global__ void fill_zero_f32(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// dq = bf16(acc * scale) over the clean then the corrupted rows
__global__ void store_dq(const float* acc, uint16_t* dq_c, uint16_t* dq_x, int64_t n_c, int64_t n,
                         float scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint16_t v = Elem<true>::from_f(acc[i] * scale);
  if (i < n_c) dq_c[i] = v;
  else dq_x[i - n_c] = v;
}

}  // namespace

hipError_t launch_dkdv_fused(const BwdArgs& a, int dtype, int d, hipStream_t s) {
  if (a.precision) return hipErrorInvalidValue;  // the default precision only
  if (a.n_kv_items <= 0) return hipSuccess;
  const dim3 grid(a.n_kv_items), block(256);
  if (dtype == BDATTN_BF16 && d == 128) hipLaunchKernelGGL((bwd_fused_kernel<true, 128, false>), grid, block, 0, s, a, nullptr);
  else if (dtype == BDATTN_BF16 && d == 32) hipLaunchKernelGGL((bwd_fused_kernel<true, 32, false>), grid, block, 0, s, a, nullptr);
  else if (dtype == BDATTN_F32 && d == 32) hipLaunchKernelGGL((bwd_fused_kernel<false, 32, false>), grid, block, 0, s, a, nullptr);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

bool bwd_fused_supported(const BwdArgs& a, int dtype, int d) {
  return dtype == BDATTN_BF16 && d == 128 && a.kv_map == nullptr && !a.precision;
}

hipError_t launch_bwd_fused(const BwdArgs& a, int dtype, int d, hipStream_t s) {
  if (!bwd_fused_supported(a, dtype, d)) return hipErrorInvalidValue;
  // the float32 dQ accumulator: one buffer per device, grown on demand and
  // kept until the process ends (a measurement path, not for concurrent use)
  static std::mutex mu;
  static std::map<int, std::pair<float*, int64_t>> bufs;
  const int64_t n = ((int64_t)a.n_clean_q + a.n_corr) * a.H * 128;
  if (n == 0) return launch_dkdv_fused(a, dtype, d, s);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  float* buf = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto& e = bufs[dev];
    if (e.second < n) {
      if (e.first) {
        (void)hipStreamSynchronize(s);
        (void)hipFree(e.first);
      }
      e = {nullptr, 0};
      if (hipMalloc(&e.first, n * sizeof(float)) != hipSuccess) return hipErrorOutOfMemory;
      e.second = n;
    }
    buf = e.first;
  }
  const int nb = int((n + 255) / 256);
  hipLaunchKernelGGL(fill_zero_f32, dim3(nb), dim3(256), 0, s, buf, n);
  if (a.n_kv_items > 0)
    hipLaunchKernelGGL((bwd_fused_kernel<true, 128, true>), dim3(a.n_kv_items), dim3(256), 0, s, a, buf);
  hipLaunchKernelGGL(store_dq, dim3(nb), dim3(256), 0, s, buf, (uint16_t*)a.dq_c, (uint16_t*)a.dq_x,
                     (int64_t)a.n_clean_q * a.H * 128, n, a.scale);
  return hipGetLastError();
}

}  // namespace bdattn
