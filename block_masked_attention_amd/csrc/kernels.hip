// gfx950 (CDNA4) kernels of block-diffusion attention.
//
// Forward and backward of the attention described in "Block Parallelism for
// Efficient Distributed Long-Context Diffusion Language Model Training":
// §3.2 gives the visibility (bdattn_mask.h), the appendix's "Efficient fused
// operator" paragraph gives the shape of the fused forward (one launch covers
// the clean-K/V part and the block-diagonal corrupted part) and of the fused
// backward (reuses saved O and LSE; returns dQ, the local corrupted dK/dV and
// the clean dK/dV summed over every local query that sees each clean key).
//
// Matrix products use the CDNA4 32x32x16 bf16 MFMA (fp32 accumulate), or, for
// fp32 problems, eight 32x32x2 fp32 MFMAs per 16-deep step. The softmax is the
// online normaliser (Milakov & Gimelshein, cited by the pages) in fp32, in
// base 2 with the scale folded into one multiply.
//
// MFMA 32x32 operand and result layout (lane l of a 64-lane wave):
//   A (32 x 16): row l%32, 8 contraction slots; B (16 x 32): column l%32,
//   8 slots. The hardware pairs slot j of A with slot j of B for the same
//   lane half (l/32); which contraction index a slot stands for is the
//   caller's choice as long as A and B agree. Here slot j of lane half h in
//   step t stands for index 16t + 8h + j ("natural"), or, when an operand is
//   built from a result tile, for 16t + 8(j/4) + 4h + j%4 ("result order").
//   C (32 x 32, 16 floats): column l%32, element i is row 8(i/4) + 4(l/32) + i%4.
// An LDS copy stored in "result order" (index bits 2 and 3 swapped within each
// 16) lets one 16-byte read supply a lane's 8 slots in either case.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bdattn_mask.h"
#include "launch.h"

namespace bdattn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float floatx2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int PAD = 8;  // elements of padding after every LDS row (bank spread)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int swap23(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ----------------------------------------------------------------- elements
template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  using T = uint16_t;  // bf16 bits
  struct Frag {
    uint4 v;
  };
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ Frag zero() { return Frag{make_uint4(0, 0, 0, 0)}; }
  static __device__ __forceinline__ Frag load(const T* p) { return Frag{*(const uint4*)p}; }
  static __device__ __forceinline__ void store(T* p, const Frag& f) { *(uint4*)p = f.v; }
  static __device__ __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    floatx2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
  // 8 floats -> 8 bf16 (round to nearest even)
  static __device__ __forceinline__ Frag pack(const float* x) {
    return Frag{make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]),
                           pack2(x[6], x[7]))};
  }
  static __device__ __forceinline__ float to_f(T v) { return __uint_as_float(uint32_t(v) << 16); }
  static __device__ __forceinline__ T from_f(float x) { return T(pack2(x, 0.f) & 0xffffu); }
  // element e (0..7) of each of 4 fragments, as 4 consecutive elements at p
  static __device__ __forceinline__ void store_col4(T* p, const Frag* f, int e) {
    const uint32_t* w0 = (const uint32_t*)&f[0].v;
    const uint32_t* w1 = (const uint32_t*)&f[1].v;
    const uint32_t* w2 = (const uint32_t*)&f[2].v;
    const uint32_t* w3 = (const uint32_t*)&f[3].v;
    const int wi = e >> 1;
    uint32_t lo, hi;
    if (e & 1) {
      lo = (w0[wi] >> 16) | (w1[wi] & 0xffff0000u);
      hi = (w2[wi] >> 16) | (w3[wi] & 0xffff0000u);
    } else {
      lo = (w0[wi] & 0xffffu) | (w1[wi] << 16);
      hi = (w2[wi] & 0xffffu) | (w3[wi] << 16);
    }
    *(uint2*)p = make_uint2(lo, hi);
  }
  static __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    *(uint2*)p = make_uint2(pack2(a, b), pack2(c, d));
  }
};

template <>
struct Elem<false> {
  using T = float;
  struct Frag {
    float4 a, b;
  };
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ Frag zero() {
    return Frag{make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)};
  }
  static __device__ __forceinline__ Frag load(const T* p) {
    return Frag{*(const float4*)p, *(const float4*)(p + 4)};
  }
  static __device__ __forceinline__ void store(T* p, const Frag& f) {
    *(float4*)p = f.a;
    *(float4*)(p + 4) = f.b;
  }
  static __device__ __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a.x, b.a.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a.y, b.a.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a.z, b.a.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a.w, b.a.w, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b.x, b.b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b.y, b.b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b.z, b.b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b.w, b.b.w, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag pack(const float* x) {
    return Frag{make_float4(x[0], x[1], x[2], x[3]), make_float4(x[4], x[5], x[6], x[7])};
  }
  static __device__ __forceinline__ float to_f(T v) { return v; }
  static __device__ __forceinline__ T from_f(float x) { return x; }
  static __device__ __forceinline__ float el(const Frag& f, int e) {
    switch (e) {
      case 0: return f.a.x;
      case 1: return f.a.y;
      case 2: return f.a.z;
      case 3: return f.a.w;
      case 4: return f.b.x;
      case 5: return f.b.y;
      case 6: return f.b.z;
      default: return f.b.w;
    }
  }
  static __device__ __forceinline__ void store_col4(T* p, const Frag* f, int e) {
    *(float4*)p = make_float4(el(f[0], e), el(f[1], e), el(f[2], e), el(f[3], e));
  }
  static __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    *(float4*)p = make_float4(a, b, c, d);
  }
};

// Row bounds of local row `row` of a query stream (0 clean, 1 corrupted).
__device__ __forceinline__ BdRowBounds row_bounds(int stream, int32_t row, int32_t clean_q_start,
                                                  const int32_t* ids, int32_t B) {
  if (stream == 0) return bd_clean_row(clean_q_start + row, B);
  return bd_corr_row(row, ids[row / B], B);
}

// ======================================================================
// Forward. One workgroup = 4 waves; wave w covers 32 query rows of one q head
// (head group: Gw heads x R rows, Gw * R / 32 = 4). It sweeps the clean keys
// [0, max cb) and then, for corrupted rows, the local corrupted keys of its
// blocks, in tiles of 64 keys staged through LDS (K as is, V transposed), double
// buffered. Per tile: S^T = K Q^T (keys x queries) so each lane owns one query
// row; mask only on tiles that need it; online softmax; O^T += V^T P^T.
// ======================================================================
template <bool BF16, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdArgs a) {
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  constexpr int TK = FWD_TK;
  constexpr int KP = D + PAD;   // K tile row pitch (elements)
  constexpr int VP = TK + PAD;  // V^T tile row pitch
  constexpr int KSZ = TK * KP, VSZ = D * VP;
  constexpr int NCH = D / 8;                 // 8-element chunks per row
  constexpr int LOADERS = (TK / 4) * NCH;    // threads that stage a tile
  static_assert(LOADERS <= 256, "tile loader needs more than 256 threads");
  static_assert(2 * (KSZ + VSZ) * E::kBytes <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) T smem[2 * (KSZ + VSZ)];

  const FwdItem it = a.items[blockIdx.x];
  const int stream = it.hs & 1, hg = it.hs >> 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, hf = lane >> 5;
  const int head = hg * a.Gw + (wave % a.Gw);
  const int kvh = head / (a.H / a.Hkv);
  const int n_rows = stream ? a.n_corr : a.n_clean_q;
  const int row0 = it.tile * a.rows_per_item;
  const int row_end = min(n_rows, row0 + a.rows_per_item);
  const int my_row = row0 + (wave / a.Gw) * 32 + lq;
  const bool row_ok = my_row < n_rows;
  const int crow = min(my_row, n_rows - 1);
  const BdRowBounds rb = row_bounds(stream, crow, a.clean_q_start, a.ids, a.B);
  const BdRowBounds first = row_bounds(stream, row0, a.clean_q_start, a.ids, a.B);
  const BdRowBounds last = row_bounds(stream, row_end - 1, a.clean_q_start, a.ids, a.B);
  const int full_end = first.cb / TK * TK;  // clean tiles below need no mask
  const int n_ct = (last.cb + TK - 1) / TK;
  const int xlo = stream ? first.xlo : 0;
  const int n_xt = stream ? (last.xhi - first.xlo + TK - 1) / TK : 0;
  const int n_tiles = n_ct + n_xt;

  const T* qsrc = (const T*)(stream ? a.q_x : a.q_c);
  const T* kc = (const T*)a.k_c;
  const T* vc = (const T*)a.v_c;
  const T* kx = (const T*)a.k_x;
  const T* vx = (const T*)a.v_x;

  // Q as the B operand of S^T = K Q^T: lane (row lq, half hf), slot j = d 16ks+8hf+j
  Frag qf[D / 16];
  {
    const T* qrow = qsrc + ((int64_t)crow * a.H + head) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = row_ok ? E::load(qrow + 16 * ks + 8 * hf) : E::zero();
  }

  // tile staging: thread -> (key group of 4, 8-element chunk)
  const int ld_c = tid % NCH, ld_g = tid / NCH;
  Frag kr[4], vr[4];
  auto fetch = [&](int j) {
    if (tid >= LOADERS) return;
    const bool cl = j < n_ct;
    const int k0 = cl ? j * TK : xlo + (j - n_ct) * TK;
    const int nk = cl ? a.n_clean_kv : a.n_corr;
    const T* ks = cl ? kc : kx;
    const T* vs = cl ? vc : vx;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k0 + 4 * ld_g + r;
      if (key < nk) {
        const int64_t off = ((int64_t)key * a.Hkv + kvh) * D + 8 * ld_c;
        kr[r] = E::load(ks + off);
        vr[r] = E::load(vs + off);
      } else {
        kr[r] = E::zero();
        vr[r] = E::zero();
      }
    }
  };
  auto stage = [&](int buf) {
    if (tid >= LOADERS) return;
    T* Ks = smem + buf * (KSZ + VSZ);
    T* Vt = Ks + KSZ;
#pragma unroll
    for (int r = 0; r < 4; ++r) E::store(Ks + (4 * ld_g + r) * KP + 8 * ld_c, kr[r]);
    const int pcol = swap23(4 * ld_g);
#pragma unroll
    for (int e = 0; e < 8; ++e) E::store_col4(Vt + (8 * ld_c + e) * VP + pcol, vr, e);
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero16();
  float m = kNegInf, l = 0.f;

  if (n_tiles > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    if (j + 1 < n_tiles) fetch(j + 1);
    const T* Ks = smem + (j & 1) * (KSZ + VSZ);
    const T* Vt = Ks + KSZ;
    const bool cl = j < n_ct;
    const int k0 = cl ? j * TK : xlo + (j - n_ct) * TK;
    const bool need_mask = !cl || (k0 + TK > full_end);

    f32x16 s[TK / 32];
#pragma unroll
    for (int mb = 0; mb < TK / 32; ++mb) {
      s[mb] = zero16();
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        Frag ka = E::load(Ks + (32 * mb + lq) * KP + 16 * ks + 8 * hf);
        E::mma(s[mb], ka, qf[ks]);
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < TK / 32; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = s[mb][i] * a.scale_log2;
        if (need_mask) {
          const int key = k0 + 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3);
          const bool vis = cl ? bd_sees_clean(rb, key) : bd_sees_corr(rb, key);
          v = vis ? v : kNegInf;
        }
        s[mb][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    float rs = 0.f;
    Frag pf[TK / 32][2];
#pragma unroll
    for (int mb = 0; mb < TK / 32; ++mb) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = exp2f(s[mb][i] - m_use);
        rs += p[i];
      }
      pf[mb][0] = E::pack(p);
      pf[mb][1] = E::pack(p + 8);
    }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
#pragma unroll
      for (int mb = 0; mb < TK / 32; ++mb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          Frag va = E::load(Vt + (32 * db + lq) * VP + 32 * mb + 16 * t + 8 * hf);
          E::mma(o[db], va, pf[mb][t]);
        }
      }
    }
    if (j + 1 < n_tiles) stage((j + 1) & 1);
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32);
  if (row_ok) {
    const float inv = 1.f / lt;
    T* orow = (T*)(stream ? a.o_x : a.o_c) + ((int64_t)my_row * a.H + head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        E::store4(orow + 32 * db + 8 * g + 4 * hf, o[db][4 * g] * inv, o[db][4 * g + 1] * inv,
                  o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      }
    }
    if (hf == 0) {
      float* lse = stream ? a.lse_x : a.lse_c;
      lse[(int64_t)head * n_rows + my_row] = (m + log2f(lt)) * kLn2;
    }
  }
}

// ======================================================================
// Backward preprocess: D = rowsum(dO * O) per (row, head), and zero the fp32
// dQ accumulator. D/8 lanes per (row, head).
// ======================================================================
template <bool BF16, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const void* o_, const void* do_, float* Dout,
                                                       float* dqa, int32_t n_rows, int32_t H) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int LPR = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = idx / LPR;
  const int sub = int(idx % LPR);
  const int64_t npairs = (int64_t)n_rows * H;
  float acc = 0.f;
  if (pair < npairs) {
    const T* o = (const T*)o_ + pair * D + 8 * sub;
    const T* g = (const T*)do_ + pair * D + 8 * sub;
    typename E::Frag fo = E::load(o), fg = E::load(g);
    const T* po = (const T*)&fo;
    const T* pg = (const T*)&fg;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += E::to_f(po[e]) * E::to_f(pg[e]);
    float* q = dqa + pair * D + 8 * sub;
    *(float4*)q = make_float4(0, 0, 0, 0);
    *(float4*)(q + 4) = make_float4(0, 0, 0, 0);
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, LPR);
  if (pair < npairs && sub == 0) {
    const int64_t row = pair / H, head = pair % H;
    Dout[head * n_rows + row] = acc;
  }
}

// fp32 dQ accumulator -> output dtype, times the softmax scale.
template <bool BF16>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* acc, void* out_, int64_t n,
                                                         float scale) {
  using E = Elem<BF16>;
  using T = typename E::T;
  T* out = (T*)out_;
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += stride) {
    float4 v = *(const float4*)(acc + i);
    E::store4(out + i, v.x * scale, v.y * scale, v.z * scale, v.w * scale);
  }
}

// ======================================================================
// Backward main. One workgroup = 4 waves owning 128 keys of one KV head (32
// per wave, kept in registers as the B operand of S = Q K^T and dP = dO V^T).
// It sweeps every query tile (64 rows) that sees its keys, for each q head of
// the group: recompute S, P = exp2(S*c - LSE2), dP, dS = P (dP - D);
// dV += P^T dO and dK += dS^T Q accumulate in registers; dQ += dS K is
// contracted over the workgroup's 128 keys through LDS and added into the
// fp32 accumulator with atomics.
// ======================================================================
template <bool BF16, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_kernel(BwdArgs a) {
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  constexpr int TK = BWD_TK, TQ = BWD_TQ;
  constexpr int NCH = D / 8;
  constexpr int KTP = TK + PAD;  // K^T rows (d) x keys
  constexpr int QP = D + PAD;    // Q, dO rows (q) x d
  constexpr int QTP = TQ + PAD;  // Q^T, dO^T rows (d) x q (result order)
  constexpr int SP = TK + PAD;   // dS rows (q) x keys
  constexpr int KT_SZ = D * KTP, Q_SZ = TQ * QP, QT_SZ = D * QTP, S_SZ = TQ * SP;
  constexpr int LDS_ELEMS = KT_SZ + 2 * Q_SZ + 2 * QT_SZ + S_SZ;
  static_assert(LDS_ELEMS * E::kBytes + TQ * 16 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) T smem[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) float r_lse2[TQ];
  __shared__ __attribute__((aligned(16))) float r_d[TQ];
  __shared__ __attribute__((aligned(16))) int32_t r_lo[TQ];
  __shared__ __attribute__((aligned(16))) int32_t r_hi[TQ];
  T* Kt = smem;
  T* Qs = Kt + KT_SZ;
  T* dOs = Qs + Q_SZ;
  T* Qt = dOs + Q_SZ;
  T* dOt = Qt + QT_SZ;
  T* dSs = dOt + QT_SZ;

  const BwdItem it = a.items[blockIdx.x];
  const int kstream = it.hs & 1, kvh = it.hs >> 1;
  const int G = a.H / a.Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lk = lane & 31, hf = lane >> 5;
  const int key0 = it.ktile * TK;
  const int n_keys = kstream ? a.n_corr : a.n_clean_kv;
  const int my_key = key0 + 32 * wave + lk;
  const bool key_ok = my_key < n_keys;
  const T* ksrc = (const T*)(kstream ? a.k_x : a.k_c);
  const T* vsrc = (const T*)(kstream ? a.v_x : a.v_c);

  // this lane's key and value as B operands (natural order over d)
  Frag kf[D / 16], vf[D / 16];
  {
    const int64_t off = ((int64_t)min(my_key, n_keys - 1) * a.Hkv + kvh) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = key_ok ? E::load(ksrc + off + 16 * ks + 8 * hf) : E::zero();
      vf[ks] = key_ok ? E::load(vsrc + off + 16 * ks + 8 * hf) : E::zero();
    }
  }
  // K^T of the workgroup's 128 keys (natural key order) for dQ = dS K
  for (int u = tid; u < (TK / 4) * NCH; u += 256) {
    const int c = u % NCH, g = u / NCH;
    Frag kr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 4 * g + r;
      kr[r] = key < n_keys ? E::load(ksrc + ((int64_t)key * a.Hkv + kvh) * D + 8 * c) : E::zero();
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) E::store_col4(Kt + (8 * c + e) * KTP + 4 * g, kr, e);
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }

  const int ld_c = tid % NCH, ld_g = tid / NCH;
  constexpr int LOADERS = (TQ / 4) * NCH;
  static_assert(LOADERS <= 256, "q tile loader");

  for (int qs = 1; qs >= 0; --qs) {
    const int r0 = qs ? it.x0 : it.c0;
    const int r1 = qs ? it.x1 : it.c1;
    if (r1 <= r0) continue;
    const int n_rows = qs ? a.n_corr : a.n_clean_q;
    const T* qsrc = (const T*)(qs ? a.q_x : a.q_c);
    const T* gsrc = (const T*)(qs ? a.do_x : a.do_c);
    const float* lse = qs ? a.lse_x : a.lse_c;
    const float* dd = qs ? a.d_x : a.d_c;
    float* dqa = qs ? a.dqa_x : a.dqa_c;
    for (int qt = (r1 - 1) / TQ; qt >= r0 / TQ; --qt) {
      const int q0 = qt * TQ;
      bool full = false;
      if (kstream == 0 && q0 >= r0 && key0 + TK <= n_keys) {
        const BdRowBounds fb = row_bounds(qs, q0, a.clean_q_start, a.ids, a.B);
        full = fb.cb >= key0 + TK;
      }
      for (int hh = 0; hh < G; ++hh) {
        const int h = kvh * G + hh;
        __syncthreads();  // previous users of the q-side LDS are done
        if (tid < LOADERS) {
          Frag qr[4], gr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = q0 + 4 * ld_g + r;
            if (row < n_rows) {
              const int64_t off = ((int64_t)row * a.H + h) * D + 8 * ld_c;
              qr[r] = E::load(qsrc + off);
              gr[r] = E::load(gsrc + off);
            } else {
              qr[r] = E::zero();
              gr[r] = E::zero();
            }
            E::store(Qs + (4 * ld_g + r) * QP + 8 * ld_c, qr[r]);
            E::store(dOs + (4 * ld_g + r) * QP + 8 * ld_c, gr[r]);
          }
          const int pcol = swap23(4 * ld_g);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            E::store_col4(Qt + (8 * ld_c + e) * QTP + pcol, qr, e);
            E::store_col4(dOt + (8 * ld_c + e) * QTP + pcol, gr, e);
          }
        }
        if (tid < TQ) {
          const int row = q0 + tid;
          if (row < n_rows) {
            const BdRowBounds b = row_bounds(qs, row, a.clean_q_start, a.ids, a.B);
            r_lse2[tid] = lse[(int64_t)h * n_rows + row] * kLog2e;
            r_d[tid] = dd[(int64_t)h * n_rows + row];
            r_lo[tid] = kstream ? b.xlo : 0;
            r_hi[tid] = kstream ? b.xhi : b.cb;
          } else {
            r_lse2[tid] = __builtin_inff();
            r_d[tid] = 0.f;
            r_lo[tid] = 0;
            r_hi[tid] = 0;
          }
        }
        __syncthreads();

        // S = Q K^T and dP = dO V^T for this wave's 32 keys (rows = queries)
        f32x16 sacc[TQ / 32], pacc[TQ / 32];
#pragma unroll
        for (int mb = 0; mb < TQ / 32; ++mb) {
          sacc[mb] = zero16();
          pacc[mb] = zero16();
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            Frag qa = E::load(Qs + (32 * mb + lk) * QP + 16 * ks + 8 * hf);
            E::mma(sacc[mb], qa, kf[ks]);
            Frag ga = E::load(dOs + (32 * mb + lk) * QP + 16 * ks + 8 * hf);
            E::mma(pacc[mb], ga, vf[ks]);
          }
        }
        Frag pa[TQ / 32][2], sa[TQ / 32][2];
#pragma unroll
        for (int mb = 0; mb < TQ / 32; ++mb) {
          float p[16], ds[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int q = 32 * mb + 8 * g + 4 * hf;
            const float4 l4 = *(const float4*)(r_lse2 + q);
            const float4 d4 = *(const float4*)(r_d + q);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
            int lo[4] = {0, 0, 0, 0}, hi[4] = {0, 0, 0, 0};
            if (!full) {
              const int4 lo4 = *(const int4*)(r_lo + q);
              const int4 hi4 = *(const int4*)(r_hi + q);
              lo[0] = lo4.x; lo[1] = lo4.y; lo[2] = lo4.z; lo[3] = lo4.w;
              hi[0] = hi4.x; hi[1] = hi4.y; hi[2] = hi4.z; hi[3] = hi4.w;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 4 * g + r;
              float pv = exp2f(sacc[mb][i] * a.scale_log2 - lv[r]);
              if (!full) pv = (key_ok && my_key >= lo[r] && my_key < hi[r]) ? pv : 0.f;
              p[i] = pv;
              ds[i] = pv * (pacc[mb][i] - dv4[r]);
            }
          }
          pa[mb][0] = E::pack(p);
          pa[mb][1] = E::pack(p + 8);
          sa[mb][0] = E::pack(ds);
          sa[mb][1] = E::pack(ds + 8);
          // dS (rows = queries, natural key order) for the workgroup's dQ
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3);
            dSs[q * SP + 32 * wave + lk] = E::from_f(ds[i]);
          }
        }
        // dV += P^T dO, dK += dS^T Q (contraction over this tile's queries)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
          for (int mb = 0; mb < TQ / 32; ++mb) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int col = 32 * mb + 16 * t + 8 * hf;
              Frag gb = E::load(dOt + (32 * db + lk) * QTP + col);
              E::mma(dv[db], pa[mb][t], gb);
              Frag qb = E::load(Qt + (32 * db + lk) * QTP + col);
              E::mma(dk[db], sa[mb][t], qb);
            }
          }
        }
        __syncthreads();  // dS complete
        // dQ[q, d] += sum over the 128 keys of dS[q, k] K[k, d]
        constexpr int NB = (TQ / 32) * (D / 32);
        for (int blk = wave; blk < NB; blk += 4) {
          const int mb = blk / (D / 32), db = blk % (D / 32);
          f32x16 acc = zero16();
#pragma unroll
          for (int ks = 0; ks < TK / 16; ++ks) {
            Frag sa2 = E::load(dSs + (32 * mb + lk) * SP + 16 * ks + 8 * hf);
            Frag kb2 = E::load(Kt + (32 * db + lk) * KTP + 16 * ks + 8 * hf);
            E::mma(acc, sa2, kb2);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = q0 + 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (row < n_rows)
              unsafeAtomicAdd(dqa + ((int64_t)row * a.H + h) * D + 32 * db + lk, acc[i]);
          }
        }
      }
    }
  }

  // write dK (times the scale) and dV for this wave's 32 keys
  T* dko = (T*)(kstream ? a.dk_x : a.dk_c);
  T* dvo = (T*)(kstream ? a.dv_x : a.dv_c);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + 32 * wave + 8 * (i >> 2) + 4 * hf + (i & 3);
      if (key < n_keys) {
        const int64_t off = ((int64_t)key * a.Hkv + kvh) * D + 32 * db + lk;
        dko[off] = E::from_f(dk[db][i] * a.scale);
        dvo[off] = E::from_f(dv[db][i]);
      }
    }
  }
}

template <bool BF16, int D>
hipError_t run_fwd(const FwdArgs& a, hipStream_t s, const KernelEvents& ev) {
  if (ev.start) hipEventRecord(ev.start, s);
  if (a.n_items > 0) {
    hipLaunchKernelGGL((fwd_kernel<BF16, D>), dim3(a.n_items), dim3(256), 0, s, a);
  }
  if (ev.stop) hipEventRecord(ev.stop, s);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t run_bwd(const BwdArgs& a, hipStream_t s, const KernelEvents& ev) {
  constexpr int LPR = D / 8;
  for (int st = 0; st < 2; ++st) {
    const int32_t n = st ? a.n_corr : a.n_clean_q;
    if (n == 0) continue;
    const int64_t threads = (int64_t)n * a.H * LPR;
    const int blocks = int((threads + 255) / 256);
    hipLaunchKernelGGL((bwd_prep_kernel<BF16, D>), dim3(blocks), dim3(256), 0, s,
                       st ? a.o_x : a.o_c, st ? a.do_x : a.do_c, st ? a.d_x : a.d_c,
                       st ? a.dqa_x : a.dqa_c, n, a.H);
  }
  if (ev.start) hipEventRecord(ev.start, s);
  if (a.n_items > 0) {
    hipLaunchKernelGGL((bwd_kernel<BF16, D>), dim3(a.n_items), dim3(256), 0, s, a);
  }
  if (ev.stop) hipEventRecord(ev.stop, s);
  for (int st = 0; st < 2; ++st) {
    const int32_t n = st ? a.n_corr : a.n_clean_q;
    if (n == 0) continue;
    const int64_t elems = (int64_t)n * a.H * D;
    const int blocks = int(std::min<int64_t>((elems / 4 + 255) / 256, 16384));
    hipLaunchKernelGGL((dq_convert_kernel<BF16>), dim3(blocks), dim3(256), 0, s,
                       st ? a.dqa_x : a.dqa_c, st ? a.dq_x : a.dq_c, elems, a.scale);
  }
  return hipGetLastError();
}

}  // namespace

bool have_kernels(int dtype, int d) {
  if (dtype == BDATTN_BF16) return d == 32 || d == 128;
  if (dtype == BDATTN_F32) return d == 32;
  return false;
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int d, hipStream_t s, const KernelEvents& ev) {
  if (dtype == BDATTN_BF16 && d == 128) return run_fwd<true, 128>(a, s, ev);
  if (dtype == BDATTN_BF16 && d == 32) return run_fwd<true, 32>(a, s, ev);
  if (dtype == BDATTN_F32 && d == 32) return run_fwd<false, 32>(a, s, ev);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, int d, hipStream_t s, const KernelEvents& ev) {
  if (dtype == BDATTN_BF16 && d == 128) return run_bwd<true, 128>(a, s, ev);
  if (dtype == BDATTN_BF16 && d == 32) return run_bwd<true, 32>(a, s, ev);
  if (dtype == BDATTN_F32 && d == 32) return run_bwd<false, 32>(a, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace bdattn
