// gfx950 (CDNA4) kernels of block-diffusion attention.
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
//   bwd_prep_kernel  D = rowsum(dO * O) and LSE * log2(e) per query row
//   bwd_dq_kernel    query-tile parallel: dQ = scale * dS K, written once
//   bwd_dkdv_kernel  key-tile parallel: dV = P^T dO, dK = scale * dS^T Q over
//                    every query tile (and q head of the KV group) that sees
//                    the keys, written once
// No kernel uses atomics, so every output is bitwise reproducible.
//
// Matrix products use the CDNA4 32x32x16 bf16 MFMA (fp32 accumulate), or, for
// fp32 problems, eight 32x32x2 fp32 MFMAs per 16-deep step. The softmax is the
// online normaliser (Milakov & Gimelshein, cited by the pages) in fp32, in
// base 2 with the scale folded into one multiply.
//
// MFMA 32x32 operand and result layout (lane l of a 64-lane wave):
//   A (32 x 16): row l%32, 8 contraction slots; B (16 x 32): column l%32,
//   8 slots. The hardware pairs slot j of A with slot j of B for the same
//   lane half h = l/32; which contraction index a slot stands for is the
//   caller's choice as long as A and B agree. Here slot j of half h in the
//   16-deep step starting at k0 stands for k0 + 8h + j ("natural"), or, when an
//   operand is built from a result tile, for k0 + 8(j/4) + 4h + j%4 ("result
//   order").
//   C (32 x 32, 16 floats): column l%32, element i is row 8(i/4) + 4h + i%4.
//
// LDS tiles are row-major with no padding; the 16-byte chunk c of row r sits
// at chunk position c ^ swz(r), swz(r) = 4(r%4) + (r/4)%4. The LDS has 64
// banks: a row-slice operand read (ds_read_b128, 16 lanes per cycle = 16
// consecutive rows, same chunk) and a transposed operand read
// (ds_read_b64_tr_b16, 32 lanes per cycle = 4 consecutive rows x 64 bytes)
// both hit 64 distinct banks. The transposed read gives lane i of each 16-lane
// group column i of four consecutive rows, i.e. the operand of a matrix whose
// contraction index runs down the tile's rows, so no transposed copy is ever
// stored.
//
// Tile loops are double buffered with the buffer index a compile-time
// constant of the loop body (two copies of each body), so every LDS operand
// read carries its buffer in the instruction's immediate offset.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bdattn_mask.h"
#include "launch.h"

namespace bdattn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float floatx2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short shortx4;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

template <int N>
using Int = std::integral_constant<int, N>;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The forward moves its running row maximum (log2 units) as soon as a tile's
// maximum exceeds it, so the largest softmax weight of a row is exactly 1
// when it is rounded to bf16 for the P V product. (Letting the maximum lag by
// a margin saves rescales but rounds the dominant weight, which the gradients
// of strongly peaked rows amplify.)
constexpr float kRescaleMargin = 0.f;

// 2^x with one v_exp_f32 (results below 2^-126 flush to zero, which is
// harmless for softmax weights; exp2(-inf) = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Chunk swizzle of row r in a tile with NCH 16-byte chunks per row.
template <int NCH>
__device__ __forceinline__ int tile_swz(int r) {
  return (((r & 3) << 2) | ((r >> 2) & 3)) & (NCH - 1);
}

// Element offset of (row r, column col) in a swizzled tile of D-element rows
// with EPC elements per 16-byte chunk.
template <int D, int EPC>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * D + (((col / EPC) ^ tile_swz<D / EPC>(r)) * EPC) + (col % EPC);
}

// ----------------------------------------------------------------- elements
template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  using T = uint16_t;  // bf16 bits
  static constexpr int EPC = 8;
  struct Frag {
    uint4 v;
  };
  static __device__ __forceinline__ Frag zero() { return Frag{make_uint4(0, 0, 0, 0)}; }
  // 8 consecutive elements from global memory
  static __device__ __forceinline__ Frag load(const T* p) { return Frag{*(const uint4*)p}; }
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
  static __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    *(uint2*)p = make_uint2(pack2(a, b), pack2(c, d));
  }
};

template <>
struct Elem<false> {
  using T = float;
  static constexpr int EPC = 4;
  struct Frag {
    float4 a, b;
  };
  static __device__ __forceinline__ Frag zero() {
    return Frag{make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)};
  }
  static __device__ __forceinline__ Frag load(const T* p) {
    return Frag{*(const float4*)p, *(const float4*)(p + 4)};
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
  static __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    *(float4*)p = make_float4(a, b, c, d);
  }
};

// Per-lane byte offsets of the operand reads from swizzled LDS tiles. The
// swizzle depends on a row's low 4 bits only, so 32-row blocks and 16-row
// steps add compile-time constants to a few offsets fixed per lane. Offsets
// are relative to the start of the kernel's LDS array; the template argument
// TILE of the reads adds the (compile-time) byte offset of the tile itself,
// buffer included.
template <bool BF16, int D>
struct OperandReads {
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  static constexpr int EPC = E::EPC;
  static constexpr uint32_t ROW = D * sizeof(T);  // bytes per tile row
  static constexpr int NCHF = BF16 ? 1 : 2;       // 16-byte chunks per fragment
  static constexpr int NTR = BF16 ? 2 : 8;         // reads per transposed fragment
  uint32_t row[D / 16][NCHF];  // row lane%32, column 16 ks + 8 (lane/32) (+4)
  uint32_t tr[D / 32][NTR];    // transposed: see tr_frag

  __device__ __forceinline__ void init(int lane) {
    const int lq = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int c = 0; c < NCHF; ++c)
        row[ks][c] = sizeof(T) * tile_off<D, EPC>(lq, 16 * ks + 8 * h + 4 * c);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      if (BF16) {
        // ds_read_b64_tr_b16: lanes r/4 = 0..3 of each 16-lane group address
        // four consecutive rows, 4 r%4 columns apart (see the file header)
        const int r = lane & 15, c = (lane >> 4) & 1;
        const int col = 32 * db + 16 * c + 4 * (r & 3);
#pragma unroll
        for (int t = 0; t < NTR; ++t)
          tr[db][t] = sizeof(T) * tile_off<D, EPC>(8 * t + 4 * h + (r >> 2), col);
      } else {
#pragma unroll
        for (int j = 0; j < NTR; ++j)
          tr[db][j] = sizeof(T) * tile_off<D, EPC>(8 * (j >> 2) + 4 * h + (j & 3), 32 * db + lq);
      }
    }
  }
  // 8 consecutive elements of row 32 mb + lane%32, from column 16 ks + 8
  // (lane/32), of the tile TILE bytes into the LDS array `lds`.
  template <uint32_t TILE>
  __device__ __forceinline__ Frag row_frag(const void* lds, int mb, int ks) const {
    const char* b = (const char*)lds + TILE + mb * 32 * ROW;
    if constexpr (BF16) {
      return Frag{*(const uint4*)(b + row[ks][0])};
    } else {
      return Frag{*(const float4*)(b + row[ks][0]), *(const float4*)(b + row[ks][1])};
    }
  }
  // Operand whose contraction index runs down the tile rows, in result order:
  // lane l takes column 32 db + l%32; slot j of half h takes row
  // k0 + 8 (j/4) + 4 h + j%4 (k0 a multiple of 16).
  template <uint32_t TILE>
  __device__ __forceinline__ Frag tr_frag(const void* lds, int k0, int db) const {
    const char* b = (const char*)lds + TILE + k0 * ROW;
    if constexpr (BF16) {
      const shortx4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(b + tr[db][0]));
      const shortx4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(b + tr[db][1]));
      const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
      return Frag{make_uint4(ux.x, ux.y, uy.x, uy.y)};
    } else {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = *(const float*)(b + tr[db][j]);
      return E::pack(x);
    }
  }
};

// Row bounds of local row `row` of a query stream (0 clean, 1 corrupted).
__device__ __forceinline__ BdRowBounds row_bounds(int stream, int32_t row, int32_t clean_q_start,
                                                  const int32_t* ids, int32_t B) {
  if (stream == 0) return bd_clean_row(clean_q_start + row, B);
  return bd_corr_row(row, ids[row / B], B);
}

// floor(n / d) for 0 <= n < 2^24, d >= 1, with inv_d = 1.0f / d: a float
// estimate that is off by at most one, then corrected with integer checks.
__device__ __forceinline__ int div_small(int n, int d, float inv_d) {
  int q = int(float(n) * inv_d);
  q -= q * d > n ? 1 : 0;
  q += (q + 1) * d <= n ? 1 : 0;
  return q;
}

// ------------------------------------------------------------ tile staging
// Tiles are copied from global memory straight into LDS (global_load_lds,
// 16 bytes per lane: lane l of the wave writes LDS bytes [base + 16 l, +16)).
// The copy is issued from inline assembly so that the compiler neither holds
// registers for it nor waits for it before unrelated LDS reads; callers wait
// with lds_dma_wait() before the barrier that publishes the tile. M0 (the LDS
// base of the copy) is saved and restored around it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base));
}

__device__ __forceinline__ void lds_dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait for every outstanding vector-memory load, visibly to the compiler.
// Register loads issued before a tile loop would otherwise stay "pending" in
// the compiler's bookkeeping at the loop header, and it would place a full
// vmcnt(0) inside the loop, where that wait also drains the (invisible)
// prefetch copies of the next tile.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Copy plan of one lane for staging R rows x D elements of a token-major
// tensor into a swizzled LDS tile with NW waves: the lane's 16-byte chunks
// and their element offsets within the source rows, computed once. Rows past
// nrows - 1 repeat row nrows - 1 (callers mask them).
template <typename T, int R, int D, int NW>
struct TileCopy {
  static constexpr int EPC = 16 / int(sizeof(T));
  static constexpr int NCH = D / EPC;
  static constexpr int NT = 64 * NW;
  static constexpr int NC = R * NCH;              // chunks in the tile
  static constexpr int CPW = (NC + NT - 1) / NT;  // copies per lane
  static_assert(NC % 64 == 0 && (NC % NT == 0 || NC < NT), "tile chunks vs workgroup size");
  uint32_t off[CPW];  // element offset of each copy's chunk: r * stride + c * EPC
  int wave, lane;
  int64_t stride;

  __device__ __forceinline__ void init(int wave_, int lane_, int64_t stride_) {
    wave = wave_;
    lane = lane_;
    stride = stride_;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int pos = u * NT + wave * 64 + lane;
      const int r = pos / NCH, c = (pos % NCH) ^ tile_swz<NCH>(r);
      off[u] = uint32_t(r * stride + c * EPC);
    }
  }
  __device__ __forceinline__ bool active() const { return !(NC < NT && wave * 64 >= NC); }
  __device__ __forceinline__ void issue(T* tile, const T* src, int row0, int nrows) const {
    if (!active()) return;  // small tile: whole waves idle
    const uint32_t base = lds_addr(tile) + uint32_t(wave * 64) * 16u;
    if (row0 + R <= nrows) {
      const T* s0 = src + (int64_t)row0 * stride;
#pragma unroll
      for (int u = 0; u < CPW; ++u)
        lds_dma16(s0 + off[u], __builtin_amdgcn_readfirstlane(base + uint32_t(u * NT) * 16u));
    } else {
#pragma unroll
      for (int u = 0; u < CPW; ++u) {
        const int pos = u * NT + wave * 64 + lane;
        const int r = pos / NCH, c = (pos % NCH) ^ tile_swz<NCH>(r);
        const int row = min(row0 + r, nrows - 1);
        lds_dma16(src + (int64_t)row * stride + c * EPC,
                  __builtin_amdgcn_readfirstlane(base + uint32_t(u * NT) * 16u));
      }
    }
  }
};

// ======================================================================
// Query-tile work item shared by the forward and the dQ kernel: `rows`
// consecutive rows of one stream for Gw q heads of one KV group; wave w covers
// 32 rows of one head. The keys are swept in tiles of TK staged through LDS
// (K and V, row-major, double buffered): the clean prefix [0, last cb), then,
// for corrupted rows, the local corrupted keys of their blocks.
// ======================================================================
struct QTile {
  int stream, head, kvh, n_rows, row0, my_row, crow, n_ct, n_xt, xlo, full_end;
  bool row_ok;
  BdRowBounds rb;
};

template <int TK>
__device__ __forceinline__ QTile q_tile(const FwdItem& it, int rows_per_item, int Gw, int H,
                                        int Hkv, int n_clean_q, int n_corr, int clean_q_start,
                                        const int32_t* ids, int B, int wave, int lq) {
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
  q.rb = row_bounds(q.stream, q.crow, clean_q_start, ids, B);
  const BdRowBounds first = row_bounds(q.stream, q.row0, clean_q_start, ids, B);
  const BdRowBounds last = row_bounds(q.stream, row_end - 1, clean_q_start, ids, B);
  q.full_end = first.cb / TK * TK;  // clean tiles below need no mask
  q.n_ct = (last.cb + TK - 1) / TK;
  q.xlo = q.stream ? first.xlo : 0;
  q.n_xt = q.stream ? (last.xhi - first.xlo + TK - 1) / TK : 0;
  return q;
}

// ======================================================================
// Forward. Per key tile: S^T = K Q^T (keys x queries, so each lane owns one
// query row); mask only on tiles that need it; online softmax; O^T += V^T P^T.
// ======================================================================
template <bool BF16, int D>
__global__ __launch_bounds__(FWD_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdArgs a) {
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
  const QTile q = q_tile<TK>(a.items[blockIdx.x], a.rows_per_item, a.Gw, a.H, a.Hkv,
                             a.n_clean_q, a.n_corr, a.clean_q_start, a.ids, a.B, wave, lq);
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

  TileCopy<T, TK, D, FWD_WAVES> cp;
  cp.init(wave, lane, (int64_t)a.Hkv * D);
  const T* const kc = (const T*)a.k_c + (int64_t)q.kvh * D;
  const T* const kx = (const T*)a.k_x + (int64_t)q.kvh * D;
  const T* const vc = (const T*)a.v_c + (int64_t)q.kvh * D;
  const T* const vx = (const T*)a.v_x + (int64_t)q.kvh * D;
  // stage key tile j (K then V) into LDS buffer `buf`
  auto fetch = [&](int j, int buf) __attribute__((always_inline)) {
    const bool cl = j < q.n_ct;
    const int k0 = cl ? j * TK : q.xlo + (j - q.n_ct) * TK;
    const int nk = cl ? a.n_clean_kv : a.n_corr;
    T* dst = smem + buf * 2 * TSZ;
    cp.issue(dst, cl ? kc : kx, k0, nk);
    cp.issue(dst + TSZ, cl ? vc : vx, k0, nk);
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

    f32x16 s[TK / 32];
#pragma unroll
    for (int mb = 0; mb < TK / 32; ++mb) {
      s[mb] = zero16();
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) E::mma(s[mb], rd.template row_frag<KT>(smem, mb, ks), qf[ks]);
    }
    // online softmax; the row max is taken on raw scores (the scale is > 0)
    // and the scale folded into the exponent's multiply-add
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < TK / 32; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (MASK) {
          const int key = k0 + 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3);
          const bool vis = cl ? bd_sees_clean(q.rb, key) : bd_sees_corr(q.rb, key);
          s[mb][i] = vis ? s[mb][i] : kNegInf;
        }
        mx = fmaxf(mx, s[mb][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
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
    Frag pf[TK / 32][2];
    float rs = 0.f;
#pragma unroll
    for (int mb = 0; mb < TK / 32; ++mb) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(fmaf(s[mb][i], a.scale_log2, -m_use));
        rs += p[i];
      }
      pf[mb][0] = E::pack(p);
      pf[mb][1] = E::pack(p + 8);
    }
    l += rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int mb = 0; mb < TK / 32; ++mb) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          E::mma(o[db], rd.template tr_frag<VT>(smem, 32 * mb + 16 * t, db), pf[mb][t]);
      }
    }
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
  if (n_tiles > 0) fetch(0, 0);
  vm_drain();
  __syncthreads();
  // tiles [0, j_full) lie inside every row's clean prefix and skip the mask
  const int j_full = min(q.n_ct, q.full_end / TK);
  sweep(std::false_type{}, 0, j_full);
  sweep(std::true_type{}, j_full, n_tiles);

  const float lt = l + __shfl_xor(l, 32);
  if (q.row_ok) {
    const float inv = 1.f / lt;
    T* orow = (T*)(q.stream ? a.o_x : a.o_c) + ((int64_t)q.my_row * a.H + q.head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        E::store4(orow + 32 * db + 8 * g + 4 * hf, o[db][4 * g] * inv, o[db][4 * g + 1] * inv,
                  o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
    }
    if (hf == 0) {
      float* lse = q.stream ? a.lse_x : a.lse_c;
      lse[(int64_t)q.head * q.n_rows + q.my_row] = (m + log2f(lt)) * kLn2;
    }
  }
}

// ======================================================================
// Backward preprocess: per (row, head) D = rowsum(dO * O) and LSE * log2(e),
// D/8 lanes each, written [H][n_pad]; rows n..n_pad-1 get D = 0, LSE = +inf
// (query tiles past the end of a stream then contribute nothing).
// ======================================================================
template <bool BF16, int D>
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
    typename E::Frag fo = E::load((const T*)o_ + pair * D + 8 * sub);
    typename E::Frag fg = E::load((const T*)do_ + pair * D + 8 * sub);
    const T* po = (const T*)&fo;
    const T* pg = (const T*)&fg;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += E::to_f(po[e]) * E::to_f(pg[e]);
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, LPR);
  if (pair < npairs && sub == 0) {
    Dout[head * n_pad + row] = real ? acc : 0.f;
    L2out[head * n_pad + row] = real ? lse[head * n_rows + row] * kLog2e : __builtin_inff();
  }
}

// ======================================================================
// Backward, dQ. Same query tiles and key sweep as the forward. Per key tile:
// S^T = K Q^T and dP^T = V dO^T (each lane owns one query row, so its LSE and
// D are scalars); P^T = exp2(S^T c - LSE2); dS^T = P^T (dP^T - D);
// dQ^T += K^T dS^T with K^T read transposed from the K tile.
// ======================================================================
template <bool BF16, int D>
__global__ __launch_bounds__(FWD_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a) {
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
  const QTile q = q_tile<TK>(a.q_items[blockIdx.x], a.rows_per_item, a.Gw, a.H, a.Hkv,
                             a.n_clean_q, a.n_corr, a.clean_q_start, a.ids, a.B, wave, lq);
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
  const float drow = q.row_ok ? (q.stream ? a.d_x : a.d_c)[ri] : 0.f;

  TileCopy<T, TK, D, FWD_WAVES> cp;
  cp.init(wave, lane, (int64_t)a.Hkv * D);
  const T* const kc = (const T*)a.k_c + (int64_t)q.kvh * D;
  const T* const kx = (const T*)a.k_x + (int64_t)q.kvh * D;
  const T* const vc = (const T*)a.v_c + (int64_t)q.kvh * D;
  const T* const vx = (const T*)a.v_x + (int64_t)q.kvh * D;
  // stage key tile j (K then V) into LDS buffer `buf`
  auto fetch = [&](int j, int buf) __attribute__((always_inline)) {
    const bool cl = j < q.n_ct;
    const int k0 = cl ? j * TK : q.xlo + (j - q.n_ct) * TK;
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
    Frag sf[TK / 32][2];
#pragma unroll
    for (int mb = 0; mb < TK / 32; ++mb) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        E::mma(s, rd.template row_frag<KT>(smem, mb, ks), qf[ks]);
        E::mma(dp, rd.template row_frag<VT>(smem, mb, ks), gf[ks]);
      }
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(fmaf(s[i], a.scale_log2, -lse2));
        if (MASK) {
          const int key = k0 + 32 * mb + 8 * (i >> 2) + 4 * hf + (i & 3);
          const bool vis = cl ? bd_sees_clean(q.rb, key) : bd_sees_corr(q.rb, key);
          p = vis ? p : 0.f;
        }
        ds[i] = p * (dp[i] - drow);
      }
      sf[mb][0] = E::pack(ds);
      sf[mb][1] = E::pack(ds + 8);
    }
#pragma unroll
    for (int mb = 0; mb < TK / 32; ++mb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          E::mma(dq[db], rd.template tr_frag<KT>(smem, 32 * mb + 16 * t, db), sf[mb][t]);
      }
    }
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
  if (n_tiles > 0) fetch(0, 0);
  vm_drain();
  __syncthreads();
  // tiles [0, j_full) lie inside every row's clean prefix and skip the mask
  const int j_full = min(q.n_ct, q.full_end / TK);
  sweep(std::false_type{}, 0, j_full);
  sweep(std::true_type{}, j_full, n_tiles);

  if (q.row_ok) {
    T* out = (T*)(q.stream ? a.dq_x : a.dq_c) + ((int64_t)q.my_row * a.H + q.head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        E::store4(out + 32 * db + 8 * g + 4 * hf, dq[db][4 * g] * a.scale,
                  dq[db][4 * g + 1] * a.scale, dq[db][4 * g + 2] * a.scale,
                  dq[db][4 * g + 3] * a.scale);
    }
  }
}

// ======================================================================
// Backward, dK/dV. One workgroup = 8 waves owning BWD_TK keys of one KV head.
// Waves w and w + 4 (which share a SIMD) own the same 32 keys, in two roles:
//   the P wave    S = Q K^T, P = exp2(S c - LSE2) (masked), dV += P^T dO;
//   the dS wave   dP = dO V^T, dS = P (dP - D), dK += dS^T Q,
// with P handed over through LDS in the exact register layout in which both
// waves hold their 32 x 32 result tiles. Each step (BWD_TQ query rows of one
// q head) has two phases separated by a barrier: {S, P | dP} then {dV | dS,
// dK}, so in each phase one wave's vector work overlaps the other's matrix
// products. Each wave keeps one accumulator (dV or dK) and one operand (K or
// V) in registers, which lets two waves share a SIMD. The next step's Q and dO
// tiles and its LSE2 / D values are copied into the other LDS buffer while the
// current one is in use. Tiles whose rows all see every key of the workgroup
// come first and skip the mask.
// ======================================================================
template <bool BF16, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdArgs a) {
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  constexpr int TK = BWD_TK, TQ = BWD_TQ, NW = 8, NMB = TQ / 32;
  constexpr int TSZ = TQ * D;
  static_assert(TK == 32 * NW / 2, "two waves per 32 keys");
  static_assert(TQ % 32 == 0 && TQ <= 128, "row data copy: one wave, 16 bytes per lane");
  __shared__ __attribute__((aligned(16))) T smem[4 * TSZ];        // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float r_row[2][2][TQ];  // [buffer][LSE2, D]
  __shared__ __attribute__((aligned(16))) float4 p_hand[NW / 2][NMB][4][64];  // P handoff
  static_assert(sizeof(smem) + sizeof(r_row) + sizeof(p_hand) <= 160 * 1024, "LDS");
  constexpr uint32_t TB = TSZ * sizeof(T);  // bytes per tile

  const BwdItem item = a.kv_items[blockIdx.x];
  const int it_x0 = item.x0, it_x1 = item.x1, it_c0 = item.c0, it_c1 = item.c1;
  const int it_xf = item.xf, it_cf = item.cf;
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
  const float inv_b = 1.f / float(a.B);
  const int key_blk = div_small(my_key, a.B, inv_b);  // clean: global block; corrupted: local

  // this lane's key (P wave) or value (dS wave) as B operand, natural over d
  Frag kvf[D / 16];
  {
    const T* src = (const T*)(p_role ? (kstream ? a.k_x : a.k_c) : (kstream ? a.v_x : a.v_c));
    const int64_t off = ((int64_t)min(my_key, n_keys - 1) * a.Hkv + kvh) * D;
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
  // starting at or after xf / cf) come first, then the ones that need the
  // mask; within each, corrupted tiles then clean ones, each from the last
  // tile down, every q head of the group per tile. A step is (tile index t in
  // that order, head offset hi), advanced without divisions.
  auto ntiles = [](int r0, int r1) { return r1 > r0 ? (r1 - 1) / TQ - r0 / TQ + 1 : 0; };
  const int top_x = (it_x1 - 1) / TQ, top_c = (it_c1 - 1) / TQ;
  const int nf_x = it_xf < it_x1 ? top_x - it_xf / TQ + 1 : 0;
  const int nf_c = it_cf < it_c1 ? top_c - it_cf / TQ + 1 : 0;
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
      s.q0 = (top_x - t) * TQ;
    } else if ((t -= nf_x) < nf_c) {
      s.qs = 0;
      s.q0 = (top_c - t) * TQ;
    } else if ((t -= nf_c) < nm_x) {
      s.qs = 1;
      s.q0 = (top_x - nf_x - t) * TQ;
    } else {
      t -= nm_x;
      s.qs = 0;
      s.q0 = (top_c - nf_c - t) * TQ;
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
  // next TQ/4 lanes D (kept opaque so the per-step stream choice stays a
  // register select rather than a load of the selected argument)
  const float* rsrc_c = lane < TQ / 4 ? a.l2_c : a.d_c;
  const float* rsrc_x = lane < TQ / 4 ? a.l2_x : a.d_x;
  asm volatile("" : "+v"(rsrc_c), "+v"(rsrc_x));
  TileCopy<T, TQ, D, NW> cp;
  cp.init(wave, lane, (int64_t)a.H * D);
  // copy step s's Q and dO tiles and its LSE2 / D rows into LDS buffer `buf`
  auto fetch = [&](const Step& s, int buf) __attribute__((always_inline)) {
    const int n_rows = s.qs ? a.n_corr : a.n_clean_q;
    const T* qsrc = (const T*)(s.qs ? a.q_x : a.q_c) + (int64_t)s.h * D;
    const T* gsrc = (const T*)(s.qs ? a.do_x : a.do_c) + (int64_t)s.h * D;
    T* dst = smem + buf * 2 * TSZ;
    cp.issue(dst, qsrc, s.q0, n_rows);
    cp.issue(dst + TSZ, gsrc, s.q0, n_rows);
    if (wave == 0 && lane < TQ / 2) {  // lanes [0, TQ/4): LSE2 of the TQ rows, then D
      constexpr int L = TQ / 4;
      const int64_t r0 = (int64_t)s.h * row_pad(n_rows) + s.q0 + 4 * (lane % L);
      const float* src = (s.qs ? rsrc_x : rsrc_c) + r0;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(&r_row[buf][0][0])));
    }
  };

  // 32 x 32 result tile of block mb of tile TILE: its rows against this
  // wave's keys, contraction over d with the operand kept in registers
  auto product = [&](auto tile_tag, int mb, f32x16& c) __attribute__((always_inline)) {
    constexpr uint32_t TILE = decltype(tile_tag)::value;
    Frag fr[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) fr[ks] = rd.template row_frag<TILE>(smem, mb, ks);
    c = zero16();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) E::mma(c, fr[ks], kvf[ks]);
  };
  // acc += X^T Y over the 32 rows of block mb, X given as packed result-order
  // fragments, Y the rows of tile TILE read transposed
  auto accumulate = [&](auto tile_tag, int mb, const Frag* x) __attribute__((always_inline)) {
    constexpr uint32_t TILE = decltype(tile_tag)::value;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      Frag y[D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) y[db] = rd.template tr_frag<TILE>(smem, 32 * mb + 16 * t, db);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) E::mma(acc[db], x[t], y[db]);
    }
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
    auto sees = [&](int row) -> bool __attribute__((always_inline)) {
      if (!key_ok || row >= n_rows) return false;
      const int rb = div_small(row, a.B, inv_b);
      if (kstream) return rb == key_blk;  // own corrupted block
      if (st.qs == 0) return key_blk <= div_small(a.clean_q_start + row, a.B, inv_b);
      return key_blk < a.ids[rb];
    };
    Frag pa[NMB][2];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      f32x16 s;
      product(QT{}, mb, s);
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
      pa[mb][0] = E::pack(p);
      pa[mb][1] = E::pack(p + 8);
    }
    __syncthreads();  // P handed over
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) accumulate(GT{}, mb, pa[mb]);
    pos = nxt;
    lds_dma_wait();
    __syncthreads();
  };
  // dS wave: dP, then (once P is there) dS = P (dP - D), dK += dS^T Q
  auto body_ds = [&](auto buf_tag, int i) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    using QT = std::integral_constant<uint32_t, BUF * 2 * TB>;
    using GT = std::integral_constant<uint32_t, BUF * 2 * TB + TB>;
    const Pos nxt = next_pos(pos);
    if (i + 1 < n_it) fetch(decode(nxt), BUF ^ 1);
    f32x16 dp[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) product(GT{}, mb, dp[mb]);
    __syncthreads();  // P handed over
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      float ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr = 32 * mb + 8 * g + 4 * hf;
        const float4 d4 = *(const float4*)(&r_row[BUF][1][qr]);
        const float4 p4 = p_hand[kg][mb][g][lane];
        ds[4 * g + 0] = p4.x * (dp[mb][4 * g + 0] - d4.x);
        ds[4 * g + 1] = p4.y * (dp[mb][4 * g + 1] - d4.y);
        ds[4 * g + 2] = p4.z * (dp[mb][4 * g + 2] - d4.z);
        ds[4 * g + 3] = p4.w * (dp[mb][4 * g + 3] - d4.w);
      }
      const Frag sa[2] = {E::pack(ds), E::pack(ds + 8)};
      accumulate(QT{}, mb, sa);
    }
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
  T* out = (T*)(p_role ? (kstream ? a.dv_x : a.dv_c) : (kstream ? a.dk_x : a.dk_c));
  const float osc = p_role ? 1.f : a.scale;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + 32 * kg + 8 * (i >> 2) + 4 * hf + (i & 3);
      if (key < n_keys) out[((int64_t)key * a.Hkv + kvh) * D + 32 * db + lk] = E::from_f(acc[db][i] * osc);
    }
  }
}

template <bool BF16, int D>
hipError_t run_fwd(const FwdArgs& a, hipStream_t s, const KernelEvents* ev) {
  if (ev) (void)hipEventRecord(ev[0].start, s);
  if (a.n_items > 0)
    hipLaunchKernelGGL((fwd_kernel<BF16, D>), dim3(a.n_items), dim3(FWD_WAVES * 64), 0, s, a);
  if (ev) (void)hipEventRecord(ev[0].stop, s);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t run_bwd(const BwdArgs& a, hipStream_t s, const KernelEvents* ev) {
  constexpr int LPR = D / 8;
  for (int st = 0; st < 2; ++st) {
    const int32_t n = st ? a.n_corr : a.n_clean_q;
    if (n == 0) continue;
    const int32_t n_pad = row_pad(n);
    const int64_t threads = (int64_t)n_pad * a.H * LPR;
    const int blocks = int((threads + 255) / 256);
    hipLaunchKernelGGL((bwd_prep_kernel<BF16, D>), dim3(blocks), dim3(256), 0, s,
                       st ? a.o_x : a.o_c, st ? a.do_x : a.do_c, st ? a.lse_x : a.lse_c,
                       st ? a.d_x : a.d_c, st ? a.l2_x : a.l2_c, n, n_pad, a.H);
  }
  if (ev) (void)hipEventRecord(ev[0].start, s);
  if (a.n_q_items > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<BF16, D>), dim3(a.n_q_items), dim3(FWD_WAVES * 64), 0, s, a);
  if (ev) (void)hipEventRecord(ev[0].stop, s);
  if (ev) (void)hipEventRecord(ev[1].start, s);
  if (a.n_kv_items > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D>), dim3(a.n_kv_items), dim3(512), 0, s, a);
  if (ev) (void)hipEventRecord(ev[1].stop, s);
  return hipGetLastError();
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

hipError_t launch_bwd(const BwdArgs& a, int dtype, int d, hipStream_t s, const KernelEvents* ev) {
  if (dtype == BDATTN_BF16 && d == 128) return run_bwd<true, 128>(a, s, ev);
  if (dtype == BDATTN_BF16 && d == 32) return run_bwd<true, 32>(a, s, ev);
  if (dtype == BDATTN_F32 && d == 32) return run_bwd<false, 32>(a, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace bdattn
