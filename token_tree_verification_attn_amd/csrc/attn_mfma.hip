// attn_mfma.hip -- matrix-core tree attention for bf16 ([SI] §4 "Tree
// Attention", "Tree-Based Parallel Decoding"; [SSD] §3 "Implementation": a
// cache part and an in-tree part, both feeding one softmax).
//
// One workgroup = NW wavefronts (4 or 8, one workgroup per CU) handles one
// (request b, kv head h, block of NW*QW packed query rows r = node*G + g,
// chunk of its key tiles: prefix tiles first, then in-tree tiles).  Per tile
// of KT keys:
//   S^T[key][query] = K Q^T     v_mfma_f32_16x16x32_bf16, A = K (LDS,
//                               ds_read_b128), B = the wave's queries (VGPRs)
//   online softmax on S^T       a query's KT scores sit in 4 lanes x KT/16
//                               registers; p = 2^(s*c - m) against the running
//                               max m, whose update (two lane swaps) is only
//                               needed when a tile would overflow a bound
//   O^T[d][query] += V^T P^T    A = V^T read from the row-major V tile with
//                               ds_read_b64_tr_b16, B = P^T straight from the
//                               S^T registers (bf16 by v_cvt_pk_bf16_f32)
// KV tiles are copied HBM -> LDS by the hardware (global_load_lds_dwordx4,
// 16 bytes per lane, no register staging) into a ring of NST stages, so the
// loads of the next tiles are in flight while the current one is computed.
// Each 16-byte chunk of a tile row is stored at an XOR-swizzled position (the
// lanes choose their source addresses accordingly), which keeps both LDS read
// patterns free of bank conflicts.
//
// Workgroups are numbered XCD-first: the dispatcher deals consecutive
// workgroups round-robin to the 8 XCDs, and the remap below gives each XCD a
// contiguous range of work items, so the row blocks that stream the same KV
// chunk run on the same XCD and share its L2.
#include <type_traits>

#include "attn_plan.h"
#include "launch.h"
#include "ttv_common.h"

#define TTV_LDS __attribute__((address_space(3)))

namespace ttv {

namespace {

constexpr float kLn2f = 0.693147180559945309f;
constexpr int kXcds = 8;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // RNE
  return __builtin_bit_cast(uint32_t, v);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | [15:14],
// expcnt[6:4] = 7 and lgkmcnt[11:8] = 15 mean "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One HBM -> LDS copy of 16 bytes per lane: lane l's 16 bytes at
// gbase + voff (gbase wave-uniform, in SGPRs; voff the lane's 32-bit offset)
// land at LDS address lds_base + 16*l (lds_base wave-uniform, passed in M0).
// It is written as inline assembly on purpose.  The compiler's memory-counter
// bookkeeping treats an LDS-DMA copy as a pending write to all of LDS, and
// before every later LDS read it cannot tell apart from the copy's target --
// the transposed V reads -- it drains every copy in flight (vmcnt(0)), which
// defeats the ring.  Issued this way the copies are ordered by the ring's own
// waits instead (wait_vmcnt for this wave's copies, then ring_barrier).
__device__ __forceinline__ void lds_dma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  const uint64_t g = reinterpret_cast<uintptr_t>(gbase);
  // readfirstlane returns int: each half goes through uint32_t, or the low
  // word would be sign-extended into the high one
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)g);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(g >> 32));
  const uint64_t gs = ((uint64_t)hi << 32) | (uint64_t)lo;
  // M0 (the LDS base) is an operand bound to that register: the compiler
  // loads it and knows it changed.  The SGPR pair is written by VALU
  // (v_readfirstlane) just before; a vector-memory read of an SGPR needs 5
  // wait states after a VALU write of it, which the compiler inserts for
  // instructions it sees but not inside inline assembly -- hence the s_nop
  // (without it the copy can take a stale base and fault).
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %1, %2" : : "{m0}"(m0), "v"(voff), "s"(gs) : "memory");
}

// Loads of the queries and parent indices, issued before the tile copies and
// also as inline assembly: the compiler would wait for a load it knows of
// with vmcnt(0) at the value's first use, which (the copies being invisible
// to it) drains every tile in flight.  wait_pin then waits for exactly these
// loads (vmcnt = the copies issued after them) in the same statement that
// hands their registers back to the compiler, so nothing reads or moves the
// registers before the data has landed (its comment names the registers, to
// check that in the assembly).  Only the address is read at issue.
__device__ __forceinline__ u32x4 gload16_async(const void* p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ int gload4_async(const void* p) {
  int v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
template <int N, int NQ>
__device__ __forceinline__ void wait_pin(u32x4 (&q)[NQ], int& p0, int& p1) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  if constexpr (NQ == 2) {
    asm volatile("s_waitcnt vmcnt(%4) ; %0 %1 %2 %3" : "+v"(q[0]), "+v"(q[1]), "+v"(p0), "+v"(p1) : "n"(N) : "memory");
  } else if constexpr (NQ == 4) {
    asm volatile("s_waitcnt vmcnt(%6) ; %0 %1 %2 %3 %4 %5"
                 : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(p0), "+v"(p1) : "n"(N) : "memory");
  } else {
    static_assert(NQ == 8, "query fragments per lane");
    asm volatile("s_waitcnt vmcnt(%10) ; %0 %1 %2 %3 %4 %5 %6 %7 %8 %9"
                 : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(q[4]), "+v"(q[5]), "+v"(q[6]),
                   "+v"(q[7]), "+v"(p0), "+v"(p1)
                 : "n"(N) : "memory");
  }
}

// Workgroup barrier for the copy ring.  __syncthreads() carries
// workgroup-scope fences, and the compiler may satisfy them by draining every
// outstanding vector-memory operation (vmcnt(0)), which would also wait for
// the tiles still in flight.  Here the caller has already waited for the
// copies that must have landed (wait_vmcnt), LDS reads are drained
// explicitly, and the compiler-only fences keep LDS accesses on their side
// of the barrier.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Reductions over the lanes l, l^16, l^32, l^48 (the four lanes that hold one
// query's scores): v_permlane16_swap / v_permlane32_swap exchange the halves
// of each 32-lane (64-lane) group in the VALU, with no LDS round trip.
// Called with the same register twice, each returns both halves' values in
// every lane (one in each result), so combining the two results reduces over
// the pair.
__device__ __forceinline__ float red16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float red32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float red16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float red32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

template <int D, int QW, int NW, int NST>
struct MfmaCfg {
  static constexpr int KT = 64;                // keys per tile
  static constexpr int kWaves = NW;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int QT = QW / 16;           // 16-query MFMA tiles per wave
  static constexpr int KS = D / 32;            // 32-wide d steps of K Q^T
  static constexpr int DT = D / 16;            // 16-wide d tiles of O^T
  static constexpr int KB = KT / 16;           // 16-key tiles per KV tile
  static constexpr int PK = KT / 32;           // 32-key steps of V^T P^T
  static constexpr int CPR = D / 8;            // 16-byte chunks per key row
  static constexpr int TILE_BYTES = KT * D * 2;        // one K (or V) tile
  static constexpr int LOADS = TILE_BYTES / 16 / kThreads;  // per thread per tile
  static constexpr int RB = kWaves * QW;       // query rows per workgroup
  // LDS: the K tiles of all stages, then the V tiles of all stages, so that
  // every stage, key-block and 32-key-step offset of the fragment reads is
  // below 64 KB of a per-lane base and fits the DS instructions' 16-bit
  // immediate (no address arithmetic in the tile loop)
  static constexpr int LDS_BYTES = NST * 2 * TILE_BYTES;
  static constexpr int V_REGION = NST * TILE_BYTES;
  // one workgroup per CU (the matrix-core shapes take up to 256 VGPRs per lane)
  static constexpr int MIN_BLOCKS = 1;
  static_assert(LOADS >= 1 && TILE_BYTES % (16 * kThreads) == 0, "tile / loads");
  static_assert(NST >= 2 && NST <= 4, "ring depth");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS per workgroup");
  static_assert(V_REGION <= 65536, "fragment read offsets must fit the 16-bit DS offset");
};

// Chunk swizzles: the physical 16-byte slot of logical chunk c of key row k.
template <int CPR>
__device__ __forceinline__ int swz_k(int key, int c) { return c ^ (key & (CPR - 1)); }
template <int CPR>
__device__ __forceinline__ int swz_v(int key, int c) { return c ^ ((key << 1) & (CPR - 1)); }

// Tile schedule of one workgroup: first nP prefix tiles (keys
// [k_begin, k_end) of k/v_cache), then nT in-tree tiles (keys from tree0*64
// on, of k/v_tree).  In-tree tiles come last so that the tree topology,
// which only they need, is built while the prefix streams.  With the split
// fixed on the host, chunk c takes the prefix keys [c*chunk, min(L,
// (c+1)*chunk)) and chunk 0 also all in-tree tiles; with the balanced split a
// chunk is a range of the unit's tile list (attn_plan.h).
struct Sched {
  int nP, k_begin, k_end, nT, tree0;
  __device__ bool tree(int t) const { return t >= nP; }
  __device__ int key0(int t) const { return t < nP ? k_begin + t * 64 : (tree0 + t - nP) * 64; }
};

template <int D, int QW, int NW, int NST>
__global__ __launch_bounds__(64 * NW, (MfmaCfg<D, QW, NW, NST>::MIN_BLOCKS)) void attn_mfma2_kernel(
    AttnArgs a, int work_items) {
  using C = MfmaCfg<D, QW, NW, NST>;
  constexpr int KT = C::KT;
  extern __shared__ __attribute__((aligned(1024))) unsigned char s_dyn[];

  // ---- XCD-first work item: rb fastest, then chunk, then (b, h)
  const int nb = gridDim.x;
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd = (nb + kXcds - 1) / kXcds;
  const int item = xcd * per_xcd + blockIdx.x / kXcds;
  if (item >= work_items) return;
  const int nrb = (a.R + C::RB - 1) / C::RB;
  int b, h, rb, c, n_chunks;
  PlanItem pl;
  if (a.balanced) {
    if (!attn_plan_item(a, item, pl)) return;
    b = pl.b;
    h = pl.h;
    rb = pl.rb;
    c = pl.c;
    n_chunks = pl.C;
  } else {
    rb = item % nrb;
    c = (item / nrb) % a.chunks;
    const int bh0 = item / (nrb * a.chunks);
    b = bh0 / a.Hkv;
    h = bh0 - b * a.Hkv;
    n_chunks = a.chunks;
  }
  const int bh = b * a.Hkv + h;

  // the wave index is wave-uniform; readfirstlane tells the compiler so, which
  // keeps the copies' LDS destinations (M0) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g16 = lane >> 4, c16 = lane & 15;
  const int N = a.N, G = a.G, R = a.R;
  const int row_base = rb * C::RB + wave * QW;
  uint16_t* out = static_cast<uint16_t*>(a.out);

  // The (request, kv head) bases come out of 64-bit products that the
  // compiler forms on the VALU; they are wave-uniform, and readfirstlane
  // puts them in scalar registers once, so that no copy needs its own.
  auto uniform = [](const char* p) {
    const uint64_t v = reinterpret_cast<uintptr_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
  };
  const char* kc = uniform(static_cast<const char*>(a.k_cache) + (size_t)bh * a.Lcap * D * 2);
  const char* vc = uniform(static_cast<const char*>(a.v_cache) + (size_t)bh * a.Lcap * D * 2);
  // the tree's K/V: their own tensors, or the cache rows after the prefix
  // (set below once the prefix length is known)
  const char* ktr = a.tree_in_cache ? kc : uniform(static_cast<const char*>(a.k_tree) + (size_t)bh * N * D * 2);
  const char* vtr = a.tree_in_cache ? vc : uniform(static_cast<const char*>(a.v_tree) + (size_t)bh * N * D * 2);

  // ---- per-lane constants of the HBM -> LDS copies.  Wave w, copy j fills
  // LDS slots (j*NW + w)*64 + lane of a tile (16 bytes each, placed by the
  // hardware at base + 16*lane); slot p holds key p / CPR, logical chunk
  // swz(key, p % CPR), i.e. this lane reads byte offset key*2D + 16*swz(...)
  // of the tile's first row.
  uint32_t koff[C::LOADS], voff[C::LOADS];
  int lkey[C::LOADS];
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int slot = (j * C::kWaves + wave) * 64 + lane;
    const int key = slot / C::CPR, phys = slot % C::CPR;
    lkey[j] = key;
    koff[j] = key * (D * 2) + swz_k<C::CPR>(key, phys) * 16;
    voff[j] = key * (D * 2) + swz_v<C::CPR>(key, phys) * 16;
  }
  // The request's prefix length (raw, for its status), its tree and this
  // wave's queries are requested first; the topology is only needed at the
  // first in-tree tile.  L is read through the scalar cache: its wait then
  // counts scalar loads only, not the tile copies issued meanwhile.  The
  // parent and query loads go out before the copies (see gload16_async);
  // lanes and rows past the end read index 0 / row 0 and are masked below.
  const int L = *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(a.cache_len + b));
  // the request's node count (rows of padding nodes get zero output)
  const int n_raw = a.n_nodes ? *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
                                    reinterpret_cast<uintptr_t>(a.n_nodes + b))
                              : N;
  const int nU = nodes_used(__builtin_amdgcn_readfirstlane(n_raw), N);
  const int32_t* par = a.parents + (size_t)b * N;
  int p0 = gload4_async(par + min(lane, N - 1));
  int p1 = gload4_async(par + min(lane + 64, N - 1));
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  u32x4 qraw[C::QT * C::KS];
  int qnode[C::QT];
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
    const int r = row_base + qt * 16 + c16;
    const bool rv = r < R;
    const int i = rv ? r / G : 0;
    qnode[qt] = rv ? i : -1;
    const int hq = h * G + (rv ? r - i * G : 0);
    const uint16_t* qr = q + (((size_t)b * N + i) * a.Hq + hq) * D + g16 * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qraw[qt * C::KS + ks] = gload16_async(qr + ks * 32);
  }
  // ---- speculative prologue (fixed split): the first ring tiles of chunk c
  // start at key c*chunk_keys whatever L is, so they are copied before L
  // arrives -- but only if they lie below Lmax (inside the cache) and inside
  // the chunk.  Once L is known, a chunk whose first tiles are not all full
  // prefix tiles drains these copies and issues its real prologue (a copy of
  // rows at or past L must not be used: those rows may hold non-finite
  // values, and a zero probability times a NaN is still a NaN).
  constexpr int kPre = NST - 1;
  const int spec_begin = a.balanced ? 0 : c * a.chunk_keys;
  const bool spec = !a.balanced && a.chunk_keys >= kPre * KT && spec_begin + kPre * KT <= a.Lmax;
  auto issue_full = [&](int key0, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    TTV_LDS unsigned char* kst = (TTV_LDS unsigned char*)(s_dyn + S * C::TILE_BYTES);
    TTV_LDS unsigned char* vst = (TTV_LDS unsigned char*)(s_dyn + C::V_REGION + S * C::TILE_BYTES);
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int wbase = (j * C::kWaves + wave) * 1024;
      lds_dma16(kc + (size_t)key0 * (D * 2), koff[j], (uint32_t)(uintptr_t)(kst + wbase));
      lds_dma16(vc + (size_t)key0 * (D * 2), voff[j], (uint32_t)(uintptr_t)(vst + wbase));
    }
  };
  if (spec) {
    issue_full(spec_begin, std::integral_constant<int, 0>{});
    if (kPre > 1) issue_full(spec_begin + KT, std::integral_constant<int, 1 % NST>{});
    if (kPre > 2) issue_full(spec_begin + 2 * KT, std::integral_constant<int, 2 % NST>{});
  }

  Sched sc;
  if (a.balanced) {  // everything is known from the plan, L (clamped) included
    const int nPtot = (pl.L + KT - 1) / KT;  // the unit's tiles: nPtot prefix, then pl.nT in-tree
    const int pe = min(pl.t1, nPtot), tt = max(pl.t0, nPtot);
    sc.nP = max(0, pe - pl.t0);
    sc.k_begin = pl.t0 * KT;
    sc.k_end = min(pl.L, sc.k_begin + sc.nP * KT);
    sc.nT = max(0, pl.t1 - tt);
    sc.tree0 = tt - nPtot;
  } else {
    // L is clamped to [0, Lmax] for the copies, so they stay inside the
    // cache even when L is invalid; such a request is rejected at the end
    // (readfirstlane: L is uniform, and the copy bases derived from it stay
    // in scalar registers)
    const int Lc = min(max(__builtin_amdgcn_readfirstlane(L), 0), a.Lmax);
    sc.k_begin = c * a.chunk_keys;
    sc.k_end = min(Lc, sc.k_begin + a.chunk_keys);
    sc.nP = (sc.k_begin < sc.k_end) ? (sc.k_end - sc.k_begin + KT - 1) / KT : 0;
    sc.nT = (c == 0) ? (nU + KT - 1) / KT : 0;
    sc.tree0 = 0;
  }
  const int ntiles = sc.nP + sc.nT;
  if (a.tree_in_cache) {  // node i at row Lc + i, Lc = L clamped to [0, Lmax] (rows < Lmax + N <= Lcap)
    const int Lc = a.balanced ? pl.L : min(max(__builtin_amdgcn_readfirstlane(L), 0), a.Lmax);
    ktr = kc + (size_t)Lc * (D * 2);
    vtr = vc + (size_t)Lc * (D * 2);
  }
  // Copies of tile t into ring stage S.  Keys past the tile's valid ones
  // re-read the last valid row (finite values; their scores are masked), so
  // no copy leaves the tensors or reads rows at or beyond the prefix length.
  auto issue = [&](int tile, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    const bool tree = sc.tree(tile);
    const int key0 = sc.key0(tile);
    const int nvalid = tree ? min(KT, nU - key0) : min(KT, sc.k_end - key0);
    const char* ks = (tree ? ktr : kc) + (size_t)key0 * (D * 2);
    const char* vs = (tree ? vtr : vc) + (size_t)key0 * (D * 2);
    TTV_LDS unsigned char* kst = (TTV_LDS unsigned char*)(s_dyn + S * C::TILE_BYTES);
    TTV_LDS unsigned char* vst = (TTV_LDS unsigned char*)(s_dyn + C::V_REGION + S * C::TILE_BYTES);
    const bool full = nvalid == KT;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      uint32_t ko = koff[j], vo = voff[j];
      if (!full) {
        const int shift = (min(lkey[j], nvalid - 1) - lkey[j]) * (D * 2);
        ko += shift;
        vo += shift;
      }
      const int wbase = (j * C::kWaves + wave) * 1024;
      lds_dma16(ks, ko, (uint32_t)(uintptr_t)(kst + wbase));
      lds_dma16(vs, vo, (uint32_t)(uintptr_t)(vst + wbase));
    }
  };


  // ---- prologue: tiles 0 .. NST-2 and the queries are in flight when the
  // loop starts.  No workgroup barrier: the ring's first one is the first.
  // (explicit stages: a loop over tile % NST here keeps the source pointers
  // in private memory, and every access to those waits on the copies)
  // The speculative copies stand if the chunk's first kPre tiles are full
  // prefix tiles from spec_begin; otherwise each wave drains them (it
  // rewrites only its own LDS slots) and issues the real ones.
  const bool spec_ok = spec && sc.k_begin == spec_begin && sc.k_end - sc.k_begin >= kPre * KT;
  if (spec && !spec_ok) wait_vmcnt<0>();
  if (!spec_ok) {
    if (ntiles > 0) issue(0, std::integral_constant<int, 0>{});
    if (kPre > 1 && ntiles > 1) issue(1, std::integral_constant<int, 1 % NST>{});
    if (kPre > 2 && ntiles > 2) issue(2, std::integral_constant<int, 2 % NST>{});
  }
  // Queries and parents have landed once no more than the prologue's copies
  // are outstanding.  One wait_pin with a fixed count (a short prologue
  // drains first): one per case would give the compiler one definition per
  // case to merge, and it merges by copying the registers before the wait.
  if (ntiles < kPre) wait_vmcnt<0>();
  wait_pin<kPre * 2 * C::LOADS>(qraw, p0, p1);
  p0 = lane < nU ? p0 : -1;
  p1 = lane + 64 < nU ? p1 : -1;
  // rows of padding nodes work on zero queries and are written as zeros
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) qnode[qt] = qnode[qt] < nU ? qnode[qt] : -1;
  bf16x8 qB[C::QT][C::KS];
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qB[qt][ks] = __builtin_bit_cast(bf16x8, qnode[qt] >= 0 ? qraw[qt * C::KS + ks] : u32x4{0u, 0u, 0u, 0u});

  // Ancestor bitsets of this lane's query nodes, built by every wave in its
  // own registers (no LDS, no barrier) when it first needs them: at the first
  // in-tree tile, or at the end for a workgroup that reports the request's
  // status without holding in-tree tiles.
  uint64_t anc_lo[C::QT], anc_hi[C::QT];
  bool tree_ok = true, tree_built = false;
  auto build_tree = [&]() {
    uint64_t a0lo, a1lo, a1hi;
    tree_ok = wave_tree_bits(p0, p1, nU, a0lo, a1lo, a1hi);
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
      const int i = qnode[qt] >= 0 ? qnode[qt] : 0;
      const uint64_t lo0 = shfl_u64(a0lo, i & 63);
      const uint64_t lo1 = shfl_u64(a1lo, i & 63);
      const uint64_t hi1 = shfl_u64(a1hi, i & 63);
      anc_lo[qt] = qnode[qt] < 0 ? 0ull : (i < 64 ? lo0 : lo1);
      anc_hi[qt] = qnode[qt] < 0 || i < 64 ? 0ull : hi1;
    }
    tree_built = true;
  };
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
    anc_lo[qt] = 0ull;
    anc_hi[qt] = 0ull;
  }
  // m_run: the running max in log2 units (-inf until the query has seen a
  // key); m_set: every query of the wave has one (wave-uniform), which
  // enables the fast softmax.
  f32x4 oacc[C::QT][C::DT];
  float m_run[C::QT], l_run[C::QT];
  bool m_set = false;
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- per-lane LDS read offsets (stage, key block and 32-key step are
  // immediates).  K: lane (c16, g16) of key block kb reads row kb*16 + c16,
  // logical chunk ks*4 + g16; its swizzle depends on c16 only.  V: see the
  // transposed read below; its swizzle depends on g16*4 + c16/4 only.
  // Each is kept as a full LDS address of stage 0 in a VGPR that the
  // compiler cannot split (the empty asm): the stage and block offsets are
  // then immediates of the reads.
  uint32_t krd[C::KS], vrd[C::DT];
  const uint32_t lds0 = (uint32_t)(uintptr_t)s_dyn;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    krd[ks] = lds0 + c16 * (D * 2) + swz_k<C::CPR>(c16, ks * 4 + g16) * 16;
    asm volatile("" : "+v"(krd[ks]));
  }
  {
    const int vkey = g16 * 4 + (c16 >> 2);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int dcol = dt * 16 + 4 * (c16 & 3);
      vrd[dt] = lds0 + C::V_REGION + vkey * (D * 2) + swz_v<C::CPR>(vkey, dcol >> 3) * 16 + ((dcol >> 2) & 1) * 8;
      asm volatile("" : "+v"(vrd[dt]));
    }
  }

  // ---- the math of one tile, in pieces.
  // Masking: bit k of tmask[qt] says whether key key0 + k is visible to this
  // lane's query (the valid-key prefix for a tail tile, the ancestor bits for
  // an in-tree tile); full prefix tiles skip it.
  // Softmax: scores stay raw until the exponent, p = 2^(s*c - m) with
  // c = scale*log2(e) > 0, so masked scores are -inf.  Fast path (every query
  // of the wave has a running max m): p against the current m without
  // looking for the tile's max; the tile stands if every lane's sum of its p
  // is at most kBound (so no p exceeds it: far from fp32 and bf16 overflow,
  // and exact after the final normalisation).  Otherwise -- the first keys a
  // query sees, or a tile that overshoots -- the slow path takes the tile's
  // max and moves m when it exceeds m by more than kLazy (log2 units),
  // rescaling O; the moved queries' largest p is then 1.
  constexpr float kLazy = 8.0f;
  constexpr float kBound = 65536.0f;  // 2^16
  const float cs = a.scale_log2;
  using KFrag = u32x4[C::KB][C::KS];
  using SAcc = f32x4[C::KB][C::QT];
  using VFrag = i16x4[C::PK][C::DT];
  using PFrag = bf16x8[C::QT][C::PK];
  // K fragments of the tile in stage S, all requested at once (one LDS
  // latency for all of them)
  auto read_k = [&](auto stage_tag, KFrag& kf) {
    constexpr int S = decltype(stage_tag)::value;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        kf[kb][ks] = *(const TTV_LDS u32x4*)(uintptr_t)(krd[ks] + S * C::TILE_BYTES + kb * 16 * (D * 2));
  };
  // S^T = K Q^T, d-step outermost so that KB*QT independent accumulations
  // sit between two MFMAs of one chain
  auto qk = [&](const KFrag& kf, SAcc& s) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int qt = 0; qt < C::QT; ++qt) s[kb][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, kf[kb][ks]);
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt)
          s[kb][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qB[qt][ks], s[kb][qt], 0, 0, 0);
      }
  };
  // V^T fragments of 32-key step k2 of the tile in stage S.
  // ds_read_b64_tr_b16 gives lane i (of its 16-lane group) element i%4 of
  // the 8-byte rows fetched by lanes 4j + i/4 of the group; lane r of group
  // g fetches V[32*k2 + 4g + r/4 (+16)][dt*16 + 4*(r%4) ..+3], so lane i
  // receives V[32*k2 + 4g + j (+16)][dt*16 + i], j = 0..3: the A operand
  // row of output column dt*16 + i for the P^T key slots.
  // With one query tile per wave all of a tile's V^T fragments are fetched
  // ahead of the MFMAs that use them; with two or more the registers run
  // short, and each 32-key step's fragments are fetched right before its
  // MFMAs.
  constexpr bool kEarlyV = C::QT == 1;
  auto read_v = [&](auto stage_tag, int k2, VFrag& vlo, VFrag& vhi) {
    constexpr int S = decltype(stage_tag)::value;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const uint32_t pa = vrd[dt] + S * C::TILE_BYTES + k2 * 32 * (D * 2);
      vlo[k2][dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TTV_LDS i16x4*)(uintptr_t)pa);
      vhi[k2][dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TTV_LDS i16x4*)(uintptr_t)(pa + 16 * (D * 2)));
    }
  };
  // Softmax of tile `tile`, in place of its scores; lane holds keys
  // kb*16 + g16*4 + e of query c16.
  auto mask_tile = [&](int tile, SAcc& s) {
    const bool tree = sc.tree(tile);
    const int key0 = sc.key0(tile);
    const int nvalid = tree ? min(KT, nU - key0) : min(KT, sc.k_end - key0);
    if (tree || nvalid < KT) {
      // the empty asm keeps this a branch taken only by tree and tail tiles
      // (if-converted, its selects would run on every tile)
      asm volatile("");
#pragma unroll
      for (int qt = 0; qt < C::QT; ++qt) {
        const uint64_t w = key0 < 64 ? anc_lo[qt] : anc_hi[qt];
        const uint64_t vmask = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1ull);
        const uint64_t tm = ((tree ? w : ~0ull) & vmask) >> (g16 * 4);  // lane keys: kb*16 + g16*4 + e
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!((tm >> (kb * 16 + e)) & 1ull)) s[kb][qt][e] = -INFINITY;
      }
    }
  };
  auto pack_p = [&](const SAcc& s, PFrag& pB) {
    // P^T operands: slots 0-3 = keys 32*k2 + g16*4 + e, 4-7 = +16
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
      for (int k2 = 0; k2 < C::PK; ++k2) {
        const u32x4 pk = {pack2(s[2 * k2][qt][0], s[2 * k2][qt][1]),
                          pack2(s[2 * k2][qt][2], s[2 * k2][qt][3]),
                          pack2(s[2 * k2 + 1][qt][0], s[2 * k2 + 1][qt][1]),
                          pack2(s[2 * k2 + 1][qt][2], s[2 * k2 + 1][qt][3])};
        pB[qt][k2] = __builtin_bit_cast(bf16x8, pk);
      }
  };
  // Fast path: p against the current max; false (and the scores lost) when
  // some lane's sum of its p exceeds the bound, after which the caller forms
  // the scores again.
  auto softmax_fast = [&](SAcc& s, PFrag& pB) -> bool {
    float psum[C::QT];
    bool over = false;
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qt][e], cs, -m_run[qt]));
          s[kb][qt][e] = p;
          ps += p;
        }
      psum[qt] = ps;
      over |= !(ps <= kBound);
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0ull) return false;
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) l_run[qt] += psum[qt];
    pack_p(s, pB);
    return true;
  };
  // Slow path: the tile's max; m moves when it exceeds m by more than kLazy.
  // Returns whether any query of the lane moved (O must then be rescaled by
  // alpha).
  auto softmax_slow = [&](SAcc& s, PFrag& pB, float (&alpha)[C::QT]) -> bool {
    bool any_rescale = false, unset = false;
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[kb][qt][e]);
      mx = red32_max(red16_max(mx));
      const float mt = mx * cs;  // this tile's max in log2 units (-inf if all masked)
      const bool move = mt > m_run[qt] + kLazy;  // false while both are -inf
      const float m_new = move ? mt : m_run[qt];
      alpha[qt] = move ? __builtin_amdgcn_exp2f(m_run[qt] - m_new) : 1.f;
      any_rescale |= move;
      m_run[qt] = m_new;
      unset |= m_new == -INFINITY;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qt][e], cs, -m_use));
          s[kb][qt][e] = p;
          ps += p;
        }
      // fp32 row sum of the unrounded probabilities (an MFMA sum of the
      // bf16-rounded P would save these adds but costs the lse ~2^-9)
      l_run[qt] = l_run[qt] * alpha[qt] + ps;
    }
    pack_p(s, pB);
    m_set = __builtin_amdgcn_ballot_w64(unset) == 0ull;
    return any_rescale;
  };
  auto rescale = [&](const float (&alpha)[C::QT], bool any) {
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) oacc[qt][dt] *= alpha[qt];
    }
  };
  // O^T += V^T P^T for the tile in stage S (V^T fragments already in vlo/vhi
  // with one query tile per wave)
  auto pv = [&](auto stage_tag, VFrag& vlo, VFrag& vhi, const PFrag& pB) {
#pragma unroll
    for (int k2 = 0; k2 < C::PK; ++k2) {
      if (!kEarlyV) read_v(stage_tag, k2, vlo, vhi);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const i16x4 lo = vlo[k2][dt], hi = vhi[k2][dt];
        const bf16x8 A = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
            lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt)
          oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pB[qt][k2], oacc[qt][dt], 0, 0, 0);
      }
    }
  };

  // ---- the pipeline: NST-1 tiles in flight during each tile's math.
  // Each wave waits for its own copies of the current tile (vmcnt counts
  // the copies issued after them), then one barrier both publishes every
  // wave's copies and proves that every wave has finished the previous
  // tile, whose stage then receives the copies of the tile NST-1 ahead.
  // The loop is unrolled by NST so that every LDS offset is an immediate.
  auto step = [&](int tile, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    const int ahead = min(NST - 2, ntiles - 1 - tile);  // tiles issued after this one
    if (ahead >= 2) wait_vmcnt<4 * C::LOADS>();
    else if (ahead == 1) wait_vmcnt<2 * C::LOADS>();
    else wait_vmcnt<0>();
    ring_barrier();
    if (tile + NST - 1 < ntiles) issue(tile + NST - 1, std::integral_constant<int, (S + NST - 1) % NST>{});
    if (tile == sc.nP) build_tree();  // the first in-tree tile
    KFrag kf;
    SAcc s;
    VFrag vlo, vhi;
    PFrag pB;
    float alpha[C::QT];
    read_k(stage_tag, kf);
    qk(kf, s);
    if (kEarlyV) {
#pragma unroll
      for (int k2 = 0; k2 < C::PK; ++k2) read_v(stage_tag, k2, vlo, vhi);
    }
    mask_tile(tile, s);
    if (!(m_set && softmax_fast(s, pB))) {
      if (m_set) {  // the tile overshot: its scores again (the stage is intact until the next barrier)
        read_k(stage_tag, kf);
        qk(kf, s);
        mask_tile(tile, s);
      }
      rescale(alpha, softmax_slow(s, pB, alpha));
    }
    pv(stage_tag, vlo, vhi, pB);
  };
  for (int tile = 0; tile < ntiles; tile += NST) {
    step(tile, std::integral_constant<int, 0>{});
    if (tile + 1 < ntiles) step(tile + 1, std::integral_constant<int, 1 % NST>{});
    if (NST > 2 && tile + 2 < ntiles) step(tile + 2, std::integral_constant<int, 2 % NST>{});
    if (NST > 3 && tile + 3 < ntiles) step(tile + 3, std::integral_constant<int, 3 % NST>{});
  }
  wait_vmcnt<0>();  // every copy has landed before the workgroup ends

  // ---- the request's status: its tree (known once built) and its length.
  // The first work item of the request reports it (and, for the combine
  // kernel, its chunk count).
  const bool writer = c == 0 && rb == 0 && h == 0;
  if (!tree_built && (n_chunks == 1 || writer)) build_tree();
  const int status = !nodes_ok(n_raw, N) ? TTV_E_SHAPE
                     : !tree_ok ? TTV_E_TREE : (L < 0 || L > a.Lmax ? TTV_E_SHAPE : TTV_OK);
  if (writer && wave == 0 && lane == 0) {
    if (a.dev_status) a.dev_status[b] = status;
    if (a.ws_nchunks) a.ws_nchunks[b] = n_chunks;
  }

  // ---- finish: the 4 lanes of a query hold disjoint key subsets of l; a
  // rejected request gets zeros (its work was done on clamped inputs)
  const bool has_work = status == TTV_OK && ntiles > 0;
  if (n_chunks == 1) {
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
      const float lt = red32_sum(red16_sum(l_run[qt]));
      const int r = row_base + qt * 16 + c16;
      if (r >= R) continue;
      const int i = r / G, hq = h * G + (r - i * G);
      uint16_t* o = out + (((size_t)b * N + i) * a.Hq + hq) * D;
      const bool real = has_work && i < nU;  // a rejected request or a padding node gets zeros
      const float inv = real ? 1.f / lt : 0.f;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const f32x4 v = oacc[qt][dt] * inv;
        *reinterpret_cast<u32x2*>(o + dt * 16 + g16 * 4) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
      }
      if (g16 == 0 && a.lse)
        a.lse[((size_t)b * N + i) * a.Hq + hq] = real ? (m_run[qt] + __log2f(lt)) * kLn2f : 0.f;
    }
    return;
  }

  // ---- split KV: write the partial -- the chunk's normalised output in
  // bf16 (half the bytes of fp32 sums; the combine kernel, bound by these
  // bytes, weights it by l * 2^(m - M)) and its m and l in fp32.  A row that
  // sees no key of the chunk has l = 0 and weight 0: stored as 0.
  // (Merging in the last-arriving workgroup would need a device-scope release
  // per workgroup, which on this chip writes back the XCD's whole L2 and was
  // measured slower than a second launch.)
  if (!has_work) return;
  uint16_t* wsb = reinterpret_cast<uint16_t*>(a.ws_acc);
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
    const float lt = red32_sum(red16_sum(l_run[qt]));
    const int r = row_base + qt * 16 + c16;
    if (r >= R) continue;
    const size_t pr = ((size_t)bh * a.chunks + c) * R + r;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const f32x4 v = oacc[qt][dt] * inv;
      *reinterpret_cast<u32x2*>(wsb + pr * D + dt * 16 + g16 * 4) =
          u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
    }
    if (g16 == 0) {
      a.ws_ml[pr * 2] = m_run[qt];
      a.ws_ml[pr * 2 + 1] = lt;
    }
  }
}

template <int D, int QW, int NW, int NST>
static hipError_t launch_cfg(const AttnArgs& a, hipStream_t s) {
  using C = MfmaCfg<D, QW, NW, NST>;
  const int nrb = (a.R + C::RB - 1) / C::RB;
  const long items = a.balanced ? (long)a.items : (long)a.B * a.Hkv * nrb * a.chunks;
  const long blocks = (items + kXcds - 1) / kXcds * kXcds;
  auto kern = attn_mfma2_kernel<D, QW, NW, NST>;
  hipError_t e = lds_limit_once(reinterpret_cast<const void*>(kern), C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(C::kThreads), C::LDS_BYTES, s, a, (int)items);
  return hipGetLastError();
}

// rows per workgroup -> shape: 64 rows = 4 waves x 16 queries, 128 = 8 x 16
// and 256 = 8 x 32; each one workgroup per CU.  Head dimension 128 takes a
// 3-stage ring (96 KB, two tiles in flight during a tile's math): on MI355X a
// fourth stage made every workload slower (long-context 1024 rows x 32768
// keys per kv head: 545 vs 523 us; 8 requests of 1024..4096 keys: 38-41 vs
// 35-36 us; 64 rows x 512 keys: 17.4 vs 15.7 us), and two stages ran as fast
// as three.
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) {
    switch (a.rows_per_block) {
      case 64: return launch_cfg<64, 16, 4, 4>(a, s);
      case 128: return launch_cfg<64, 16, 8, 4>(a, s);
      default: return launch_cfg<64, 32, 8, 4>(a, s);
    }
  }
  switch (a.rows_per_block) {
    case 64: return launch_cfg<128, 16, 4, 3>(a, s);
    case 128: return launch_cfg<128, 16, 8, 3>(a, s);
    default: return launch_cfg<128, 32, 8, 3>(a, s);
  }
}

}  // namespace ttv
