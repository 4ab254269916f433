// Device ops of librs for gfx950 (CDNA4): KV store, extend attention, prefix-aware
// decode attention, log-sum-exp merge.
//
// The attention computed is causal softmax attention over each request's context,
// reached through its index-table row ("How does SGLang work",
// modernaiengineering.com: "A quick recap ..." -- a token's KV depends only on its
// prefix and decode appends its own KV; "What happens when a request arrives" --
// the unmatched suffix is prefilled attending to the reused KV as if it had just
// been computed).
//
// bf16 attention runs on two MFMA tile engines with one operand scheme.  K and V rows are
// gathered through the index table into LDS tiles; per tile, on 32x32x16 bf16 MFMAs:
//     S^T[key][row] = K[key][:] . Q[row][:]      (A = K from LDS, B = Q^T in registers)
//     O^T[d][row]  += V^T[d][key] . P^T[key][row] (A = V^T from LDS, B = P^T in registers)
// With S^T in the accumulator a lane holds the scores of one query row for half the
// keys (its partner lane l^32 holds the other half), so softmax bookkeeping is
// lane-local plus one cross-half exchange, and P^T feeds the second MFMA from the same
// registers: the key order that transposing LDS reads give V^T matches the accumulator.
// * decode: 4 waves of 32 rows (requests x heads), 64-key tiles, online softmax with a
//   lazily moved reference point;
// * extend: 4 waves of 64 rows (tokens x heads) in two row blocks, 32-key tiles, a
//   software-pipelined loop and exponentials of the raw scaled scores (no reference point
//   unless a row's range calls for one).
// fp32 extend runs the same operand scheme on 32x32x2 fp32 MFMAs with operands loaded
// straight into registers (workgroups of 32 query rows, 4 waves splitting the keys); fp32
// decode runs on the VALU (one wave per query row).

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>
#include <utility>

#include "internal.h"
#include "plan.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.f;   // softmax weights stay below 2^kSlack between rescales

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ uint16_t f2bf(float a) { return uint16_t(pack_bf16(a, 0.f) & 0xffffu); }

// Max / sum of v over lanes l and l ^ 32.  v_permlane32_swap exchanges the upper half of
// one operand with the lower half of the other; with v in both, the two results hold v of
// lanes l and l ^ 32 (in some order), without a round trip through LDS.
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One stage of a K/V tile in LDS: KB rows (keys) of K and of V, D*2 bytes each, unpadded.
// Rows arrive straight from global memory with global_load_lds_dwordx4: one instruction
// moves kRowsPerInst whole rows (lane l writes 16 bytes at M0 + 16*l), every lane with
// its own 64-bit source address -- a fully coalesced request, no staging registers.
//
// Two permutations make this work with the 64 x 4-byte LDS banks:
// * rows: instruction g of wave w fills LDS rows (KB/4)w + kRowsPerInst*g + j (j < rows
//   per instruction), holding keys (KB/4)w + g + kInstPerWave*j, so a lane's kInstPerWave
//   slot ids are consecutive table entries (one load) -- key_of_row() undoes it for masks;
// * 16-byte chunks: chunk c of LDS row R sits at position c ^ swz(R), which spreads the
//   16 rows of a K-operand ds_read_b128 phase and the 4 rows x 4 chunks of a V-operand
//   transposing ds_read_b64 phase over distinct banks (no conflicts).
template <int D, int KB, int NW = 4>
struct StageLayout {
  static_assert(KB == 32 || KB == 64, "tiles of 32 or 64 keys");
  static constexpr int kRow = D * 2;                  // bytes per row (K and V)
  static constexpr int kChunks = kRow / 16;           // 16-byte chunks per row
  static constexpr int kRowsPerInst = 64 / kChunks;   // rows one dwordx4 DMA instruction fills
  static constexpr int kRowsPerWave = KB / NW;        // rows each of the NW waves loads
  static constexpr int kInstPerWave = kRowsPerWave / kRowsPerInst;
  static_assert(kInstPerWave >= 1, "a wave's rows fill whole DMA instructions");
};

template <int D, int KB>
struct __align__(16) Stage {
  char k[KB * StageLayout<D, KB>::kRow];
  char v[KB * StageLayout<D, KB>::kRow];
};

template <int D>
__device__ __forceinline__ int swz(int R) {
  return D == 128 ? 4 * (R & 3) + ((R >> 2) & 3) : 4 * ((R >> 1) & 1) + ((R >> 2) & 3);
}

template <int D, int KB>
__device__ __forceinline__ int key_of_row(int R) {
  using L = StageLayout<D, KB>;
  const int rw = R % L::kRowsPerWave;
  return R - rw + rw / L::kRowsPerInst + L::kInstPerWave * (rw % L::kRowsPerInst);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Slot ids for this lane's DMA rows of the tile at key0: s[g] = slot of key
// key0 + 16w + kInstPerWave*j + g (j = lane / chunks per row).  Keys past k1 repeat the
// slot of key k1-1 -- an in-bounds row whose scores the caller masks.
template <int D, int KB>
struct TileSlots {
  int s[StageLayout<D, KB>::kInstPerWave];
};

template <int D, int KB>
__device__ __forceinline__ TileSlots<D, KB> wave_slots(const int32_t* __restrict__ trow, int key0, int k1, int wave_u,
                                                       int lane) {
  using L = StageLayout<D, KB>;
  TileSlots<D, KB> t;
  const int base = key0 + wave_u * L::kRowsPerWave;
  const int k = base + L::kInstPerWave * (lane / L::kChunks);
  // one vector load per lane when every row is in range and the entries are aligned for it
  if (L::kInstPerWave > 1 && base + L::kRowsPerWave <= k1 &&
      (reinterpret_cast<uintptr_t>(trow + base) & (4 * L::kInstPerWave - 1)) == 0) {
    typedef int slots_vec __attribute__((ext_vector_type(L::kInstPerWave > 1 ? L::kInstPerWave : 2)));
    const slots_vec v = *reinterpret_cast<const slots_vec*>(trow + k);
#pragma unroll
    for (int g = 0; g < L::kInstPerWave; ++g) t.s[g] = v[g];
  } else {
#pragma unroll
    for (int g = 0; g < L::kInstPerWave; ++g) t.s[g] = trow[min(k + g, k1 - 1)];
  }
  return t;
}

// Cache-policy operand of the load builtins: non-temporal.  Decode reads every KV byte once
// per launch (a shared segment once for all the requests that share it); its launches that
// stream at least kDecodeNtBytes of KV take the non-temporal policy (measured: 7 % faster on
// 3.2 GB, 1-3 % on 210 MB, 1.7 % slower on 45 MB).
constexpr int kCpolNT = 2;
constexpr int64_t kDecodeNtBytes = int64_t(128) << 20;

// Issue the global->LDS loads of one tile (this wave's KB/4 rows of K and of V); NT: with
// the non-temporal policy.
// co[g] = this lane's byte offset within its row for instruction g (its swizzled chunk).
template <int D, int KB, bool NT>
__device__ __forceinline__ void issue_tile(Stage<D, KB>& dst, const char* kp, const char* vp, uint32_t row_bytes,
                                           const TileSlots<D, KB>& ts,
                                           const uint32_t (&co)[StageLayout<D, KB>::kInstPerWave], int wave_u) {
  using L = StageLayout<D, KB>;
#pragma unroll
  for (int g = 0; g < L::kInstPerWave; ++g) {
    const uint64_t off = uint64_t(uint32_t(ts.s[g])) * row_bytes + co[g];
    const int r0 = wave_u * L::kRowsPerWave + g * L::kRowsPerInst;
    __builtin_amdgcn_global_load_lds(kp + off, (lds_ptr)(dst.k + r0 * L::kRow), 16, 0, NT ? kCpolNT : 0);
    __builtin_amdgcn_global_load_lds(vp + off, (lds_ptr)(dst.v + r0 * L::kRow), 16, 0, NT ? kCpolNT : 0);
  }
}

// ------------------------------------------------------------------ per-wave math
// Online-softmax state of one wave: lane l owns query row l%32 (shared with lane l^32).
template <int D>
struct WaveState {
  f32x16 o[D / 32];     // O^T accumulators: o[mb][j] = O[row][mb*32 + 8*(j/4) + 4*(lane/32) + j%4]
  float m;              // reference point of the exponentials, in raw score units: at most
                        // kSlack/c below the running max (-inf before any visible key)
  float l;              // this lane's half of the running sum of exp2((s - m) * c)
};

template <int D>
__device__ __forceinline__ void wave_init(WaveState<D>& ws) {
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int j = 0; j < 16; ++j) ws.o[mb][j] = 0.f;
  ws.m = -INFINITY;
  ws.l = 0.f;
}

// Query fragments (B operand of S^T): qf[ks] = Q[row][16*ks + 8*(lane/32) .. +8].
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[D / 16], const uint16_t* __restrict__ qrow, bool valid,
                                       int lane) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 u = valid ? *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * (lane >> 5)) : make_uint4(0, 0, 0, 0);
    qf[ks] = __builtin_bit_cast(bf16x8, u);
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// The steps of one KB-key tile for one wave (the math runs over LDS rows; the key of a
// row only matters for the mask):
//   qk:          S^T = K . Q^T                      (MFMA, K from LDS)
//   mask_scores: -inf where key >= nk or key_pos0 + key > lim (lim = the row's last
//                visible position)
//   row_max:     max over the tile of each query row (both lane halves)
//   update_ref:  move the reference point of the exponentials if needed (rescales O, l)
//   weights:     P^T = exp2(S*c - m*c) packed to bf16, and the row sums of those weights
//   pv:          O^T += V^T . P^T                   (MFMA, V^T from LDS)
// c = sm_scale*log2(e); slack = kSlack / c (the same margin in raw score units).
template <int KB>
struct Scores {
  f32x16 s[KB / 32];
};

template <int KB>
struct Weights {
  uint4 p[KB / 16];       // P^T in bf16 pairs, one B operand per 16 keys
};

template <int D, int KB>
__device__ __forceinline__ void qk(Scores<KB>& sc, const Stage<D, KB>& sm, const bf16x8 (&qf)[D / 16], int lane) {
  using L = StageLayout<D, KB>;
  const int r32 = lane & 31, hi = lane >> 5;
  const char* kb = sm.k + r32 * L::kRow;                 // LDS row r32 (and r32 + 32)
  const int fk = swz<D>(r32);                            // rows r32, r32 + 32 share it
#pragma unroll
  for (int kb32 = 0; kb32 < KB / 32; ++kb32) {
#pragma unroll
    for (int j = 0; j < 16; ++j) sc.s[kb32][j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      // elements 16ks + 8hi .. +8 of the row = 16-byte chunk 2ks + hi
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + kb32 * 32 * L::kRow + 16 * ((2 * ks + hi) ^ fk));
      sc.s[kb32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sc.s[kb32], 0, 0, 0);
    }
  }
}

template <int D, int KB>
__device__ __forceinline__ void mask_scores(Scores<KB>& sc, int lane, int nk, int key_pos0, int lim) {
  const int hi = lane >> 5;
#pragma unroll
  for (int kb32 = 0; kb32 < KB / 32; ++kb32)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = key_of_row<D, KB>(kb32 * 32 + 8 * (j >> 2) + 4 * hi + (j & 3));
      if (t >= nk || key_pos0 + t > lim) sc.s[kb32][j] = -INFINITY;
    }
}

template <int KB>
__device__ __forceinline__ float row_max(const Scores<KB>& sc) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb32 = 0; kb32 < KB / 32; ++kb32)
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc.s[kb32][j]);
  return fmaxf(mx, __shfl_xor(mx, 32));
}

// The reference point m of the exponentials moves only when some row's maximum exceeds
// it by more than kSlack (in exp2 units), so weights stay below 2^kSlack and most tiles
// skip the rescale of O and l; softmax does not depend on the point.
template <int D>
__device__ __forceinline__ void update_ref(WaveState<D>& ws, float mx, float c, float slack) {
  if (__builtin_amdgcn_ballot_w64(mx > ws.m + slack)) {
    const float m_new = fmaxf(ws.m, mx);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    // v_exp_f32 directly: results below 2^-126 flush to zero, which softmax weights can afford
    const float alpha = __builtin_amdgcn_exp2f((ws.m - m_ref) * c);
    ws.l *= alpha;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) ws.o[mb][j] *= alpha;
    ws.m = m_new;
  }
}

__device__ __forceinline__ float ref_times_c(float m, float c) { return (m == -INFINITY ? 0.f : m) * c; }

// Returns this lane's half of the row sum of the weights as the second MFMA sees them (bf16).
template <int KB>
__device__ __forceinline__ float weights(Weights<KB>& w, const Scores<KB>& sc, float c, float mc) {
  const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
  float sum = 0.f;
#pragma unroll
  for (int kstep = 0; kstep < KB / 16; ++kstep) {
    const int kb32 = kstep >> 1, h8 = (kstep & 1) * 8;
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(sc.s[kb32][h8 + i], c, -mc));
    w.p[kstep].x = pack_bf16(e[0], e[1]);
    w.p[kstep].y = pack_bf16(e[2], e[3]);
    w.p[kstep].z = pack_bf16(e[4], e[5]);
    w.p[kstep].w = pack_bf16(e[6], e[7]);
    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.p[kstep].x), kOnes, sum, false);
    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.p[kstep].y), kOnes, sum, false);
    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.p[kstep].z), kOnes, sum, false);
    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.p[kstep].w), kOnes, sum, false);
  }
  return sum;
}

// V^T operand by transposing LDS reads: within each 16-lane group, lane i receives
// element i%4 of the 8-byte pieces read by lanes i/4 + 4k (k = 0..3).  Provider lane j
// reads row rbase + j/4 at d = dbase + 4*(j%4), so receiver lane i gets
// V[rbase + k][dbase + i], k = 0..3: the four rows of its P^T slots 4r..4r+3.
template <int D, int KB>
__device__ __forceinline__ void pv(WaveState<D>& ws, const Stage<D, KB>& sm, const Weights<KB>& w, int lane) {
  using L = StageLayout<D, KB>;
  const int hi = lane >> 5, i16 = lane & 15, gpar = (lane >> 4) & 1;
  // this lane's rows hi*4 + i16/4 (+8, +16*kstep) at bytes 32gpar + 8(i16%4) + 64mb:
  // chunk 2gpar + (i16%4)/2 + 4mb, half i16%2; the swizzle depends on the row mod 16
  const int vr0 = hi * 4 + (i16 >> 2);
  const int cv = 2 * gpar + ((i16 & 3) >> 1);
  const int fv0 = swz<D>(vr0), fv1 = swz<D>(vr0 + 8);
  const char* vb0 = sm.v + vr0 * L::kRow + 8 * (i16 & 1);
  const char* vb1 = vb0 + 8 * L::kRow;
#pragma unroll
  for (int kstep = 0; kstep < KB / 16; ++kstep) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, w.p[kstep]);
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const char* p0 = vb0 + kstep * 16 * L::kRow + 16 * ((cv + 4 * mb) ^ fv0);
      const char* p1 = vb1 + kstep * 16 * L::kRow + 16 * ((cv + 4 * mb) ^ fv1);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
      const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
      const bf16x8 a = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
          lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
      ws.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, ws.o[mb], 0, 0, 0);
    }
  }
}

// All steps of one tile in order.
template <int D, int KB>
__device__ __forceinline__ void wave_tile(WaveState<D>& ws, const Stage<D, KB>& sm, const bf16x8 (&qf)[D / 16],
                                          int lane, bool mask, int nk, int key_pos0, int lim, float c, float slack) {
  Scores<KB> sc;
  qk<D, KB>(sc, sm, qf, lane);
  if (mask) mask_scores<D, KB>(sc, lane, nk, key_pos0, lim);   // wave-uniform: ragged or diagonal tiles
  update_ref<D>(ws, row_max<KB>(sc), c, slack);
  Weights<KB> w;
  const float sum = weights<KB>(w, sc, c, ref_times_c(ws.m, c));
  pv<D, KB>(ws, sm, w, lane);
  ws.l += sum;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Stream keys [k0, k1) of one index-table row through the workgroup, NS LDS stages deep.
// Waves with has_rows run the math (SKIP_EMPTY) or every wave does (a wave past the last
// token then has only masked rows, which contribute exact zeros); every wave issues loads.
// Keys below mask_from are visible to every row; tiles reaching past it (and a ragged
// last tile) take the masked path.
//
// Pipeline: at the top of iteration t the workgroup waits for tile t (this wave's loads,
// then a barrier for everyone's, after which every wave is also done with the stage tile
// t-1 used); it then issues the slot ids of tile t+NS and the loads of tile t+NS-1 into
// that stage, and computes tile t.  While tile t+1 is in flight the wait leaves exactly
// the loads issued after tile t's (one iteration's worth) outstanding.
template <int D, int KB>
struct StreamArgs {
  const char* kc;
  const char* vc;
  const int32_t* trow;
  uint32_t row_bytes;
  uint32_t co[StageLayout<D, KB>::kInstPerWave];   // this lane's swizzled chunk offset per DMA instruction
  int k0, k1, ntiles, mask_from, lim, wave_u, lane;
  float c, slack;
  bool has_rows;
};

// Iteration t of the pipeline; its tile sits in stage t % NS.
template <int D, int KB, int NS, bool SKIP_EMPTY, bool NT>
__device__ __forceinline__ void stream_step(WaveState<D>& ws, Stage<D, KB> (&sm)[NS], const bf16x8 (&qf)[D / 16],
                                            const StreamArgs<D, KB>& a, TileSlots<D, KB>& s_next, int t) {
  using L = StageLayout<D, KB>;
  // K + V DMA and the next slot loads (one vector load, or kInstPerWave single loads):
  // at least this many per iteration
  constexpr int kPerIter = 2 * L::kInstPerWave + 1;
  const int key0 = a.k0 + t * KB;
  const int nk = min(KB, a.k1 - key0);
  // After tile t's loads came, in order: the next tiles' (issued one iteration each, at
  // least kPerIter instructions per iteration) -- exactly when all of them exist.
  // (vmcnt counts to 63: a smaller count only waits a little longer)
  constexpr int kAfter = (NS - 2) * kPerIter < 63 ? (NS - 2) * kPerIter : 63;
  if (NS > 2 && t + NS - 2 < a.ntiles && t >= NS - 2) wait_vmcnt_barrier<kAfter>();
  else wait_vmcnt_barrier<0>();
  if (t + NS - 1 < a.ntiles) {
    issue_tile<D, KB, NT>(sm[(t + NS - 1) % NS], a.kc, a.vc, a.row_bytes, s_next, a.co, a.wave_u);
    s_next = wave_slots<D, KB>(a.trow, a.k0 + (t + NS) * KB, a.k1, a.wave_u, a.lane);
  }
  if (!SKIP_EMPTY || a.has_rows) {
    const bool mask = nk < KB || key0 + KB > a.mask_from;
    wave_tile<D, KB>(ws, sm[t % NS], qf, a.lane, mask, nk, key0, a.lim, a.c, a.slack);
  }
}


template <int D, int KB, int NS, bool SKIP_EMPTY, bool NT>
__device__ __forceinline__ void stream_keys(WaveState<D>& ws, Stage<D, KB> (&sm)[NS], const bf16x8 (&qf)[D / 16],
                                            const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                                            const int32_t* __restrict__ trow, int Hkv, int k0, int k1,
                                            int mask_from, int lim, float c, bool has_rows, int tid) {
  if (k0 >= k1) return;
  using L = StageLayout<D, KB>;
  StreamArgs<D, KB> a;
  a.kc = reinterpret_cast<const char*>(kp);
  a.vc = reinterpret_cast<const char*>(vp);
  a.trow = trow;
  a.row_bytes = uint32_t(Hkv) * D * 2;
  a.lane = tid & 63;
  a.wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  // this lane's source byte offset within its row for each DMA instruction: the chunk
  // that belongs at its LDS position (the swizzle depends on the LDS row mod 16)
#pragma unroll
  for (int g = 0; g < L::kInstPerWave; ++g)
    a.co[g] = 16u * uint32_t((a.lane % L::kChunks) ^
                             swz<D>(a.wave_u * L::kRowsPerWave + g * L::kRowsPerInst + a.lane / L::kChunks));
  a.k0 = k0;
  a.k1 = k1;
  a.ntiles = (k1 - k0 + KB - 1) / KB;
  a.mask_from = mask_from;
  a.lim = lim;
  a.c = c;
  a.slack = kSlack / c;
  a.has_rows = has_rows;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < a.ntiles)
      issue_tile<D, KB, NT>(sm[j], a.kc, a.vc, a.row_bytes, wave_slots<D, KB>(trow, k0 + j * KB, k1, a.wave_u, a.lane),
                        a.co, a.wave_u);
  TileSlots<D, KB> s_next = wave_slots<D, KB>(trow, k0 + (NS - 1) * KB, k1, a.wave_u, a.lane);
  for (int t = 0; t < a.ntiles; ++t) stream_step<D, KB, NS, SKIP_EMPTY, NT>(ws, sm, qf, a, s_next, t);
}

// ------------------------------------------------------------------ extend (bf16)
// Extend engine.  Each wave owns 64 query rows as two 32-row blocks, and every K and V
// operand it reads from LDS feeds the MFMAs of both blocks, so LDS reads per flop are
// half those of a 32-row wave.  A workgroup is 4 waves (256 rows) and a CU holds one: each
// wave has a SIMD and up to 512 registers to itself.  The draft-tree verify instantiation
// gives each wave one 32-row block (128 rows per workgroup): its few verify tokens per
// request would leave half of a 256-row workgroup empty, and the empty rows would still
// cost their matrix and vector work.  The Q fragments and the O
// accumulators stay in AGPRs (only MFMAs touch them in the loop); the scores, weights and
// addresses use the VGPRs.
//
// Tiles of 32 keys stream through kExtNS LDS stages, kExtNS - 2 tiles ahead of the math.
// Their slot ids reach LDS the same way (a small ring filled one DMA per wave per tile,
// further ahead still), so every load in the loop goes global -> LDS and the waits count
// exactly.
//
// The loop is software-pipelined by one tile so that one wave overlaps its own matrix
// and vector work.  Iteration t: S(t) = K(t) Q^T runs on the matrix cores while the VALU
// turns S(t-1) into weights; then O += V(t-1)^T P(t-1), among whose MFMAs S(t) moves from
// the MFMA result registers to VGPRs (the copy is the pipeline's buffer swap); on the causal
// diagonal or a ragged end it is then masked.
//
// Softmax reference.  Softmax does not depend on the reference point subtracted from the
// scores before the exponential, and fp32 and bf16 carry a weight with the same relative
// precision anywhere between their common underflow near 2^-126 and overflow near 2^128.
// The first pass therefore subtracts nothing: a weight is exp2(S c) (one multiply before
// the exponential instead of a three-operand fma), the loop never rescales O and tracks
// no maximum.  Two things can spoil that: an overflow, which leaves an inf or a NaN in O
// or l, and a row whose weights are all tiny, whose small products with small values
// would fall below fp32's normal range; the output check catches both (l below 2^-40
// stands for the second: the largest weight is then below 2^-40 too).  The workgroup then
// finds each row's true maximum in a pass that tracks it and recomputes its rows with that
// maximum as the reference (every weight <= 1, the largest one 1).
constexpr int kExtKB = 32;           // keys per tile
constexpr int kExtNS = 8;            // LDS stages (16 KiB each at d128)
constexpr int kExtRows = 256;        // query rows per workgroup of the causal kernel: 4 waves x 64
constexpr int kVerifyRows = 128;     // of the draft-tree verify kernel: 4 waves x 32
constexpr int kExtAhead = kExtNS - 2;            // tiles in flight ahead of the math
// Slot ids reach LDS in groups: one 64-lane dword DMA per wave brings its kExtKB/NW ids of
// kExtRingGroup<NW> consecutive tiles, one group kExtRingGroup iterations before its first
// use, into a ring of two groups.
template <int NW>
constexpr int kExtRingGroup = 64 / (kExtKB / NW);
static_assert(kExtRingGroup<4> > kExtAhead - 1 && kExtRingGroup<8> > kExtAhead - 1, "slot group too small");

// RB: 32-row blocks per wave (2 in the causal kernel, 1 in the verify kernel).
template <int D, int RB>
struct ExtState {
  f32x16 o[RB][D / 32];         // O^T per row block (layout as WaveState)
  float mc[RB];                 // reference point times c, per row block (recompute pass)
  float mx[RB];                 // this lane's running maximum of raw scores (tracking pass)
  float l[RB];                  // this lane's halves of the running sums
};

template <int RB>
struct ExtWeights {
  uint4 p[RB][kExtKB / 16];      // [row block][16-key step]: P^T in bf16 pairs
};

// Per-lane LDS byte offsets of the MFMA operands within a stage: K chunk of step ks for
// row r32, and the two transposing-read pieces of V for output block mb.  The swizzle is
// fixed per lane, so these are computed once.
template <int D>
struct ExtOffsets {
  uint32_t k[D / 16];
  uint32_t v0[D / 32], v1[D / 32];
};

template <int D>
__device__ __forceinline__ ExtOffsets<D> ext_offsets(int lane) {
  using L = StageLayout<D, kExtKB>;
  ExtOffsets<D> off;
  const int r32 = lane & 31, hi = lane >> 5, i16 = lane & 15, gpar = (lane >> 4) & 1;
  const int fk = swz<D>(r32);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) off.k[ks] = r32 * L::kRow + 16 * ((2 * ks + hi) ^ fk);
  const int vr0 = hi * 4 + (i16 >> 2), cv = 2 * gpar + ((i16 & 3) >> 1);
  const int fv0 = swz<D>(vr0), fv1 = swz<D>(vr0 + 8);
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    off.v0[mb] = vr0 * L::kRow + 8 * (i16 & 1) + 16 * ((cv + 4 * mb) ^ fv0);
    off.v1[mb] = (vr0 + 8) * L::kRow + 8 * (i16 & 1) + 16 * ((cv + 4 * mb) ^ fv1);
  }
  return off;
}

// K fragments of one tile (A operands of S^T = K Q^T), read once for both row blocks.
template <int D>
struct KFrags {
  bf16x8 a[D / 16];
};

template <int D>
__device__ __forceinline__ KFrags<D> ext_read_k(const char* kst, const ExtOffsets<D>& off) {
  KFrags<D> f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) f.a[ks] = *reinterpret_cast<const bf16x8*>(kst + off.k[ks]);
  return f;
}

// S^T of both row blocks (results in the MFMA's accumulation registers).
template <int D, int RB>
__device__ __forceinline__ void ext_qk(f32x16 (&sc)[RB], const KFrags<D>& kf, const bf16x8 (&qf)[RB][D / 16]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int j = 0; j < 16; ++j) sc[rb][j] = 0.f;
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      sc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.a[ks], qf[rb][ks], sc[rb], 0, 0, 0);
}

// Key index within the tile of score element j (lane half 0; half 1 adds 4).
__device__ __forceinline__ constexpr int ext_key(int j) { return 8 * (j >> 2) + (j & 3); }

__device__ __forceinline__ float max16(const f32x16& v) {
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = fmaxf(m, v[j]);
  return m;
}

// Weights P = bf16(exp2(S*c)) of both row blocks (REF: bf16(exp2(S*c - m*c)) with the
// reference m) and their row sums (of the bf16 weights, as the second MFMA sees them);
// TRACK: also the running maxima of the scores.
template <int D, int RB, bool TRACK, bool REF>
__device__ __forceinline__ void ext_weights(ExtWeights<RB>& w, ExtState<D, RB>& es, const f32x16 (&sc)[RB], float c) {
  const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (TRACK) es.mx[rb] = fmaxf(es.mx[rb], max16(sc[rb]));
    float sum = 0.f;
#pragma unroll
    for (int kstep = 0; kstep < kExtKB / 16; ++kstep) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        e[i] = __builtin_amdgcn_exp2f(REF ? fmaf(sc[rb][8 * kstep + i], c, -es.mc[rb]) : sc[rb][8 * kstep + i] * c);
      uint4& p = w.p[rb][kstep];
      p.x = pack_bf16(e[0], e[1]);
      p.y = pack_bf16(e[2], e[3]);
      p.z = pack_bf16(e[4], e[5]);
      p.w = pack_bf16(e[6], e[7]);
      sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p.x), kOnes, sum, false);
      sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p.y), kOnes, sum, false);
      sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p.z), kOnes, sum, false);
      sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p.w), kOnes, sum, false);
    }
    es.l[rb] += sum;
  }
}

// V^T fragments of one tile (A operands of O^T += V^T P^T), by transposing LDS reads.
template <int D>
struct VFrags {
  bf16x8 a[kExtKB / 16][D / 32];
};

template <int D>
__device__ __forceinline__ VFrags<D> ext_read_v(const char* vst, const ExtOffsets<D>& off) {
  using L = StageLayout<D, kExtKB>;
  VFrags<D> f;
#pragma unroll
  for (int kstep = 0; kstep < kExtKB / 16; ++kstep)
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const char* p0 = vst + off.v0[mb] + kstep * 16 * L::kRow;
      const char* p1 = vst + off.v1[mb] + kstep * 16 * L::kRow;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
      const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
      f.a[kstep][mb] = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
          lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
    }
  return f;
}

// O^T += V^T P^T for both row blocks.
template <int D, int RB>
__device__ __forceinline__ void ext_pv(ExtState<D, RB>& es, const VFrags<D>& vf, const ExtWeights<RB>& w) {
#pragma unroll
  for (int kstep = 0; kstep < kExtKB / 16; ++kstep)
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        es.o[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.a[kstep][mb], __builtin_bit_cast(bf16x8, w.p[rb][kstep]),
                                                               es.o[rb][mb], 0, 0, 0);
}

template <int D, int NW>
struct ExtStream {
  const char* kc;             // K pool at this KV head
  const char* vc;
  const int32_t* trow;        // index-table row
  uint32_t row_bytes;
  uint32_t co[StageLayout<D, kExtKB, NW>::kInstPerWave];   // this lane's swizzled chunk offset per DMA instruction
  int k1, ntiles, mask_from, wave_u, lane;
  int jrow;                   // this lane's row within a DMA instruction
  int hik;                    // 4 in the upper lane half: its score elements sit 4 keys later
  int lim[2];                 // last visible key position of this lane's row per block (-1: none)
  float c;                    // sm_scale * log2(e)
  // draft-tree verify: keys at and past tree_base are visible to a row only where its
  // ancestor mask has their bit (key - tree_base); tree = false: plain causal
  bool tree;
  int tree_base;
  uint64_t tm[2];
};

// LDS of the extend workgroup: the K/V stages and the slot-id ring.
template <int D, int NW>
struct ExtShared {
  Stage<D, kExtKB> st[kExtNS];
  int32_t ring[NW][2 * kExtRingGroup<NW>][kExtKB / NW];   // per wave and tile: its slot ids
};

// Global -> LDS loads issued through inline assembly.  The LDS address goes through M0,
// set in the same statement.  The compiler does not see these as LDS writes, so it adds
// no waits of its own before later LDS reads (it would wait for every load in flight);
// each wait on them is explicit instead: the loop's vmcnt wait and barrier.  Nor do they
// clobber memory: the LDS they write is read only after a later wait-and-barrier
// statement, which orders every memory access, so LDS reads may move around them.
// (M0 is a reserved register: the compiler warns about it in a clobber list, yet nothing
// else in the extend kernel reads M0, and the clobber keeps it from assuming otherwise.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(uintptr_t((__attribute__((address_space(3))) const void*)(p)));
}

// NT: with the non-temporal cache policy, for bytes the launch reads only once.
template <bool NT>
__device__ __forceinline__ void dma_b128(const void* src, uint32_t lds) {   // lane l -> lds + 16*l
  if (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds) : "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "m0");
}

__device__ __forceinline__ void dma_b32(const void* src, uint32_t lds) {    // lane l -> lds + 4*l
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds) : "m0");
}
#pragma clang diagnostic pop

// Slot ids of tile group k (tiles kG .. kG+G-1, G = kExtRingGroup) into this wave's half of
// the ring: lane l loads the id of key kExtKB (kG + l / P) + P wave + l % P (P = kExtKB / NW,
// the wave's keys of a tile); keys past k1 repeat the last slot.
template <int D, int NW>
__device__ __forceinline__ void ext_slot_dma(ExtShared<D, NW>& sh, const ExtStream<D, NW>& a, int k) {
  constexpr int P = kExtKB / NW, G = kExtRingGroup<NW>;
  const int x = k * G + a.lane / P;
  const int32_t* src = a.trow + min(x * kExtKB + a.wave_u * P + a.lane % P, a.k1 - 1);
  dma_b32(src, lds_addr(&sh.ring[a.wave_u][(k & 1) * G][0]));
}

// This lane's slot id for each of its DMA instructions of tile x, from the ring.
template <int D, int NW>
struct ExtRowSlots {
  int s[StageLayout<D, kExtKB, NW>::kInstPerWave];
};

template <int D, int NW>
__device__ __forceinline__ ExtRowSlots<D, NW> ext_read_slots(const ExtShared<D, NW>& sh, const ExtStream<D, NW>& a, int x) {
  using L = StageLayout<D, kExtKB, NW>;
  ExtRowSlots<D, NW> r;
#pragma unroll
  for (int g = 0; g < L::kInstPerWave; ++g) r.s[g] = sh.ring[a.wave_u][x % (2 * kExtRingGroup<NW>)][g * L::kRowsPerInst + a.jrow];
  return r;
}

// Global -> LDS loads of this wave's K and V rows of one tile (NT: non-temporal).
template <int D, int NW, bool NT>
__device__ __forceinline__ void ext_kv_dma(Stage<D, kExtKB>& dst, const ExtStream<D, NW>& a, const ExtRowSlots<D, NW>& sl) {
  using L = StageLayout<D, kExtKB, NW>;
#pragma unroll
  for (int g = 0; g < L::kInstPerWave; ++g) {
    const uint64_t off = uint64_t(uint32_t(sl.s[g])) * a.row_bytes + a.co[g];
    const int r0 = a.wave_u * L::kRowsPerWave + g * L::kRowsPerInst;
    dma_b128<NT>(a.kc + off, lds_addr(dst.k + r0 * L::kRow));
    dma_b128<NT>(a.vc + off, lds_addr(dst.v + r0 * L::kRow));
  }
}

// Waits on the K/V loads, each this wave's vmcnt count and then a barrier for everyone's.
// Tiles 0 .. kExtAhead-1 are issued in order by the prologue, tile kExtAhead by the tile-0
// step and tile t + kExtAhead by iteration t, each as 2*kInstPerWave loads (past the last
// tile they reload its last row into a stage nobody reads), and loads complete in issue
// order.  So when tile x is awaited while tiles up to x + kExtAhead - 2 have been issued,
// exactly kExtAfter loads came after it (slot-id loads among them only make the wait
// longer), whatever x.
template <int D, int NW>
constexpr int kExtAfter = (kExtAhead - 2) * 2 * StageLayout<D, kExtKB, NW>::kInstPerWave;

// The tile-0 step needs tiles 0 and 1 (it reads tile 1's K ahead); tiles 2 .. kExtAhead-1
// came after them.
template <int D, int NW>
__device__ __forceinline__ void ext_wait_first() {
  static_assert(kExtAfter<D, NW> < 64, "vmcnt is 6 bits");
  wait_vmcnt_barrier<kExtAfter<D, NW>>();
}

// Iteration t (t >= 1) needs tile t + 1 (its K is read ahead, at the end of the iteration);
// tiles up to t + kExtAhead - 1 have been issued.
template <int D, int NW>
__device__ __forceinline__ void ext_wait_next() {
  wait_vmcnt_barrier<kExtAfter<D, NW>>();
}

// -inf in the scores of tile t past this lane's last visible key or the tile's last key (and,
// for the draft-tree verify, outside the row's ancestor mask).
template <int D, int RB, int NW>
__device__ __forceinline__ void ext_mask(f32x16 (&sc)[RB], const ExtStream<D, NW>& a, int t) {
  const int key0 = t * kExtKB;
  const int nk = min(kExtKB, a.k1 - key0);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int thr = min(a.lim[rb] - key0, nk - 1) - a.hik;
    if (a.tree) {
      // key k = key0 + hik + ext_key(j): causal bound as above, and past tree_base only
      // the keys of the row's ancestor mask
      const int rel0 = key0 + a.hik - a.tree_base;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int rel = rel0 + ext_key(j);
        const bool in_tree = rel < 0 || (rel < 64 && ((a.tm[rb] >> (rel & 63)) & 1));
        if (ext_key(j) > thr || !in_tree) sc[rb][j] = -INFINITY;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (ext_key(j) > thr) sc[rb][j] = -INFINITY;
    }
  }
}

// Iteration t (t >= 1): on entry prev holds S(t-1) (masked), kf
// K(t) and vf V(t-1); on exit cur holds S(t), kf K(t+1) and vf V(t).  S(t) runs on the
// matrix cores while the VALU turns S(t-1) into weights, then O += V(t-1)^T P(t-1).  The
// next K and V are read at the end, after the MFMAs are issued, so their LDS latency
// overlaps the matrix work instead of delaying the next iteration's first MFMA.
template <int D, int RB, bool MASK, bool TRACK, bool REF, int NW, bool NT>
__device__ __forceinline__ void ext_iter(ExtState<D, RB>& es, ExtShared<D, NW>& sh, const ExtOffsets<D>& off,
                                         const bf16x8 (&qf)[RB][D / 16], const ExtStream<D, NW>& a,
                                         const f32x16 (&prev)[RB], f32x16 (&cur)[RB], KFrags<D>& kf, VFrags<D>& vf,
                                         int t) {
  ext_wait_next<D, NW>();
  const ExtRowSlots<D, NW> sl = ext_read_slots<D, NW>(sh, a, t + kExtAhead);
  // the slot-id group that tile t + kExtAhead + G starts, if it starts one; it overwrites
  // the group of tiles t + kExtAhead - G .. t + kExtAhead - 1, whose last ids were read in
  // the iteration before
  constexpr int G = kExtRingGroup<NW>;
  if ((t + kExtAhead) % G == 0) ext_slot_dma<D, NW>(sh, a, (t + kExtAhead) / G + 1);
  ext_kv_dma<D, NW, NT>(sh.st[(t + kExtAhead) % kExtNS], a, sl);
  ext_qk<D, RB>(cur, kf, qf);
  ExtWeights<RB> w;
  ext_weights<D, RB, TRACK, REF>(w, es, prev, a.c);
  ext_pv<D, RB>(es, vf, w);
  kf = ext_read_k<D>(sh.st[(t + 1) % kExtNS].k, off);
  vf = ext_read_v<D>(sh.st[t % kExtNS].v, off);
  if (MASK) ext_mask<D, RB, NW>(cur, a, t);
  __builtin_amdgcn_iglp_opt(0);   // interleave the MFMAs with the other work of the body
}

// Iterations [t_begin, t_end), t_begin >= 1; sprev holds S(t_begin - 1) on entry and
// S(t_end - 1) on exit.  (Unrolling by two so that two score buffers trade roles saves no
// instruction: the scores come out of the MFMAs in accumulation registers and are moved to
// VGPRs for the vector unit either way.)
template <int D, int RB, bool MASK, bool TRACK, bool REF, int NW, bool NT>
__device__ __forceinline__ void ext_iters(ExtState<D, RB>& es, ExtShared<D, NW>& sh, const ExtOffsets<D>& off,
                                          const bf16x8 (&qf)[RB][D / 16], const ExtStream<D, NW>& a,
                                          f32x16 (&sprev)[RB], KFrags<D>& kf, VFrags<D>& vf, int t_begin, int t_end) {
  for (int t = t_begin; t < t_end; ++t) {
    f32x16 scur[RB];
    ext_iter<D, RB, MASK, TRACK, REF, NW, NT>(es, sh, off, qf, a, sprev, scur, kf, vf, t);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sprev[rb] = scur[rb];
  }
}

// One pass over keys [0, k1).  REF: es.mc holds each row's reference point; otherwise the
// weights are taken against none.  TRACK: es.mx gathers each lane's maximum score.
// ring_ready: this wave's first two slot-id groups have landed already.  NT: K/V loads with
// the non-temporal cache policy.
template <int D, int RB, bool TRACK, bool REF, int NW, bool NT>
__device__ __forceinline__ void ext_pass(ExtState<D, RB>& es, ExtShared<D, NW>& sh, const ExtOffsets<D>& off,
                                         const bf16x8 (&qf)[RB][D / 16], const ExtStream<D, NW>& a, bool ring_ready) {
  // tiles from t_mask on hold keys at or past mask_from: the causal diagonal, the ragged end
  const int t_mask = min(a.mask_from / kExtKB, a.ntiles);
  // prologue: the first two slot-id groups (the loop loads group k + 1 in the iteration
  // that reads the first ids of group k), then the K/V of the first tiles
  if (!ring_ready) {
    ext_slot_dma<D, NW>(sh, a, 0);
    ext_slot_dma<D, NW>(sh, a, 1);
    wait_vmcnt_barrier<0>();
  } else {
    // issued with the queries, which the caller has waited for already: this wave's own
    // ring rows (no other wave reads them), whatever order the loads went out in
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  for (int x = 0; x < kExtAhead; ++x) ext_kv_dma<D, NW, NT>(sh.st[x], a, ext_read_slots<D, NW>(sh, a, x));
  // tile 0: its scores only
  ext_wait_first<D, NW>();
  f32x16 sprev[RB];
  KFrags<D> kf;
  VFrags<D> vf;
  {
    const ExtRowSlots<D, NW> sl = ext_read_slots<D, NW>(sh, a, kExtAhead);
    kf = ext_read_k<D>(sh.st[0].k, off);
    ext_kv_dma<D, NW, NT>(sh.st[kExtAhead % kExtNS], a, sl);
    f32x16 scur[RB];
    ext_qk<D, RB>(scur, kf, qf);
    // tiles 0 and 1 have landed (the wait above): tile 1's K and tile 0's V for the
    // first iteration
    kf = ext_read_k<D>(sh.st[1 % kExtNS].k, off);
    vf = ext_read_v<D>(sh.st[0].v, off);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sprev[rb] = scur[rb];
    if (t_mask == 0) ext_mask<D, RB, NW>(sprev, a, 0);
  }
  const int t_split = max(1, t_mask);
  ext_iters<D, RB, false, TRACK, REF, NW, NT>(es, sh, off, qf, a, sprev, kf, vf, 1, t_split);
  ext_iters<D, RB, true, TRACK, REF, NW, NT>(es, sh, off, qf, a, sprev, kf, vf, t_split, a.ntiles);
  // the last tile's weights and P.V (vf holds its V)
  ExtWeights<RB> w;
  ext_weights<D, RB, TRACK, REF>(w, es, sprev, a.c);
  ext_pv<D, RB>(es, vf, w);
  // the loads past the last tile have landed, and every wave is done with the stages and
  // the ring, before a later pass refills them or the workgroup ends
  wait_vmcnt_barrier<0>();
}

// Zero O and l; no maximum seen yet.
template <int D, int RB>
__device__ __forceinline__ void ext_reset(ExtState<D, RB>& es) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) es.o[rb][mb][j] = 0.f;
    es.l[rb] = 0.f;
    es.mx[rb] = -INFINITY;
  }
}

// Write the valid rows' outputs O / l (bf16).  Returns true if any of them, or l, is not
// finite -- only an overflow of the weights makes that happen (x * 0 is 0 for finite x and
// NaN for inf or NaN, so z is NaN exactly then; four sums keep the chains short) -- or if
// some valid row's l is below 2^-40 (weights taken against no reference, all tiny).
// Lanes l and l ^ 32 hold the same row's d .. d+3 and d+4 .. d+7 of each 8-value group:
// one v_permlane32_swap per register pair gives each lane 16 contiguous bytes of the
// row (the lower lane the even group of a pair, the upper lane the odd one), so every
// store writes 16 bytes per lane instead of 8 -- half the store instructions.
template <int D, int RB>
__device__ __forceinline__ bool ext_store(const ExtState<D, RB>& es, const bool (&valid)[RB], const int64_t (&qrow_idx)[RB],
                                          uint16_t* __restrict__ out, int lane) {
  const int hi = lane >> 5;
  float z[4] = {0.f, 0.f, 0.f, 0.f};
  bool tiny = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!valid[rb]) continue;
    const float l = xhalf_sum(es.l[rb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    z[0] = fmaf(l, 0.f, z[0]);
    tiny |= l < 0x1p-40f;
    uint16_t* orow = out + qrow_idx[rb] * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        uint32_t w[2][2];          // [group of the pair][dword]: this lane's 4 values of d + 8 q4 + 4 hi
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int q4 = 2 * pr + h;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = es.o[rb][mb][4 * q4 + e] * inv;
            z[e] = fmaf(v[e], 0.f, z[e]);
          }
          w[h][0] = pack_bf16(v[0], v[1]);
          w[h][1] = pack_bf16(v[2], v[3]);
        }
        // upper half of w[0] <-> lower half of w[1]: the lower lane then holds group 2pr
        // (its own values, then its partner's), the upper lane group 2pr+1
        uint4 u;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const auto r = __builtin_amdgcn_permlane32_swap(w[0][c], w[1][c], false, false);
          (c == 0 ? u.x : u.y) = r[0];
          (c == 0 ? u.z : u.w) = r[1];
        }
        *reinterpret_cast<uint4*>(orow + mb * 32 + 16 * pr + 8 * hi) = u;
      }
  }
  return tiny || (z[0] + z[1]) + (z[2] + z[3]) != 0.f;   // true for NaN
}

// The rows of one workgroup (RB 32-row blocks per wave, row = 32 (RB wave + block) + lane
// % 32, tokens-major: token row / G, query head row % G of the KV head's group), their
// passes over the keys and their outputs.
template <int D, bool TREE, int NW, int RB>
__device__ __forceinline__ void ext_rows(ExtShared<D, NW>& sh, ExtStream<D, NW>& a, const uint16_t* __restrict__ q,
                                         uint16_t* __restrict__ out, const uint64_t* __restrict__ tree_mask, int wave,
                                         int lane, int G, int Hq, int kvh, int qo, int t0, int ntok) {
  bf16x8 qf[RB][D / 16];
  int64_t qrow_idx[RB];
  bool valid[RB];
  // The first slot-id groups go out before the queries: the wait for the queries below
  // (they are needed in AGPRs) then covers them too, one memory round trip for both.
  ext_slot_dma<D, NW>(sh, a, 0);
  ext_slot_dma<D, NW>(sh, a, 1);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wave * 32 * RB + rb * 32 + (lane & 31);
    const int t = row / G, g = row % G;
    valid[rb] = t < ntok;
    qrow_idx[rb] = int64_t(qo + t0 + t) * Hq + kvh * G + g;
    // A row past the tile's last token takes that token's query (its output is never
    // stored and its scores only need to be finite), so every load is unconditional and
    // they all go out together.
    load_q<D>(qf[rb], q + (int64_t(qo + t0 + min(t, ntok - 1)) * Hq + kvh * G + g) * D, true, lane);
    a.lim[rb] = valid[rb] ? a.tree_base + t0 + t : -1;
    a.tm[rb] = (a.tree && valid[rb]) ? tree_mask[qo + t0 + t] : 0ull;
  }
  const ExtOffsets<D> off = ext_offsets<D>(lane);
  ExtState<D, RB> es;
  ext_reset<D, RB>(es);
  // Q fragments and O accumulators live in AGPRs through the loop: only MFMAs read
  // them there, which leaves the VGPRs to the scores, weights and addresses.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+a"(qf[rb][ks]));
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) asm volatile("" : "+a"(es.o[rb][mb]));
  }
  // The draft-tree verify reads each request's keys once per KV head (one workgroup holds
  // all its verify tokens): those loads take the non-temporal policy.  A causal q-tile
  // shares its request's prefix with the request's other q-tiles, which find it in the
  // caches when they run together; its loads keep the default policy.
  ext_pass<D, RB, false, false, NW, TREE>(es, sh, off, qf, a, true);
  if (__syncthreads_or(ext_store<D, RB>(es, valid, qrow_idx, out, lane))) {
    // A weight overflowed or some row's weights are all tiny: find each row's true maximum,
    // then recompute the rows with it as the reference (the outputs above are overwritten).
    ext_reset<D, RB>(es);
    ext_pass<D, RB, true, false, NW, TREE>(es, sh, off, qf, a, false);
    float mx[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mx[rb] = xhalf_max(es.mx[rb]);
    ext_reset<D, RB>(es);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) es.mc[rb] = (mx[rb] == -INFINITY ? 0.f : mx[rb]) * a.c;
    ext_pass<D, RB, false, true, NW, TREE>(es, sh, off, qf, a, false);
    ext_store<D, RB>(es, valid, qrow_idx, out, lane);
  }
}

// TREE: draft-tree verify (tree_mask gives each row's ancestor mask); otherwise causal.
// NW waves per workgroup: 4 (one per SIMD; 64 rows each in the causal kernel, 32 in the
// verify kernel) or 8 (two per SIMD, 32 rows each).  The launchers use 4: on the mixed
// batch the 8-wave form is 4% slower, with the same matrix-core busy cycles and the same
// cycles of vector and matrix work overlapping, and more time waiting on dependencies.
template <int D, bool TREE, int NW, int RB>
__global__ void __launch_bounds__(64 * NW, 1) extend_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpool, const uint16_t* __restrict__ vpool,
    const int32_t* __restrict__ req_to_token, int64_t ld, const int32_t* __restrict__ qo_indptr,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ extend_lens, int n_qtiles, int Hq,
    int Hkv, float sm_scale, const int32_t* __restrict__ order, uint16_t* __restrict__ out, int uniform_n,
    const uint64_t* __restrict__ tree_mask, int defer_last) {
  static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");
  static_assert(RB == 1 || RB == 2, "32-row blocks per wave");
  constexpr int kRows = NW * 32 * RB;                // rows per workgroup (the launcher sizes the grid by it)
  __shared__ ExtShared<D, NW> sh;
  using L = StageLayout<D, kExtKB, NW>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = Hq / Hkv;
  const int tpb = kRows / G;                      // tokens per tile
  const int kvh = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  // Requests in the given order; within a request the later (longer) q-tiles first.  With
  // defer_last, every request's last q-tile (short: the launcher sets it when the longest
  // request's last tile fits the one-block loop) waits until all full q-tiles have started,
  // so the cheap workgroups fill the end of the launch.
  int qt, i;
  const int nfull = defer_last ? n_qtiles - 1 : n_qtiles;
  const int ph1 = int(gridDim.x) / Hkv / n_qtiles * nfull;
  if (rest < ph1) {
    qt = nfull - 1 - rest % nfull;
    i = rest / nfull;
  } else {
    qt = n_qtiles - 1;
    i = rest - ph1;
  }
  const int b = order ? order[i] : i;
  // uniform_n > 0: every request computes uniform_n tokens, packed in request order
  const int ext = uniform_n > 0 ? uniform_n : extend_lens[b];
  const int t0 = qt * tpb;
  if (t0 >= ext) return;
  const int prefix = prefix_lens[b];
  const int qo = uniform_n > 0 ? b * uniform_n : qo_indptr[b];
  const int ntok = min(tpb, ext - t0);
  ExtStream<D, NW> a;
  a.tree = TREE;
  a.tree_base = prefix;
  a.kc = reinterpret_cast<const char*>(kpool + int64_t(kvh) * D);
  a.vc = reinterpret_cast<const char*>(vpool + int64_t(kvh) * D);
  a.trow = req_to_token + int64_t(b) * ld;
  a.row_bytes = uint32_t(Hkv) * D * 2;
  a.lane = lane;
  a.wave_u = __builtin_amdgcn_readfirstlane(wave);
  a.jrow = lane / L::kChunks;
  a.hik = 4 * (lane >> 5);
#pragma unroll
  for (int g = 0; g < L::kInstPerWave; ++g)
    a.co[g] = 16u * uint32_t((lane % L::kChunks) ^ swz<D>(a.wave_u * L::kRowsPerWave + g * L::kRowsPerInst + a.jrow));
  a.k1 = prefix + t0 + ntok;
  a.ntiles = (a.k1 + kExtKB - 1) / kExtKB;
  a.mask_from = a.tree ? prefix : prefix + t0 + 1;   // keys below this are visible to every row
  a.c = sm_scale * kLog2e;
  // A request's last q-tile may hold few tokens.  When its rows fit in one 32-row block
  // per wave, the workgroup runs the one-block loop: half the matrix and vector work per
  // key tile for the same keys (the rows past the tile's tokens would be all masked).
  if constexpr (!TREE && RB == 2) {
    if (ntok * G <= NW * 32) {
      ext_rows<D, TREE, NW, 1>(sh, a, q, out, tree_mask, wave, lane, G, Hq, kvh, qo, t0, ntok);
      return;
    }
  }
  ext_rows<D, TREE, NW, RB>(sh, a, q, out, tree_mask, wave, lane, G, Hq, kvh, qo, t0, ntok);
}

// ------------------------------------------------------------------ decode (bf16)
// Decode: kDecKB-key tiles through kDecNS LDS stages (kDecNS - 1 tiles in flight while one
// is computed), up to two workgroups per CU.  Measured on the small decode batches and the
// mixed batch: 32-key tiles through 4 or 5 stages (more bytes in flight, twice the waits and
// barriers per key) are 4-10% slower than 64-key tiles through 2; the same work items run on
// the extend engine's pipeline (8 stages of 32 keys, 6 in flight, one workgroup per CU, which
// streams the long verify batch at 71% of HBM bandwidth) are 3-38% slower.
constexpr int kDecKB = 64, kDecNS = 2;
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kpool;
  const uint16_t* vpool;
  const int32_t* req_to_token;
  int64_t ld;
  const int32_t* seq_lens;
  const int32_t* items;       // plan: items [n_items][kItemWords]; nullptr: the flat mode
  const int4* item_req;       // plan: {request, partial index, partials of the request, -}
  const int32_t* part_ptr;    // plan: request b's partials are part_ptr[b] .. part_ptr[b+1]-1
  int flat_nch;               // flat mode: chunks per request; request b's partials b*flat_nch + chunk
  int max_seq;                // flat mode: keys are read up to min(seq_lens[b], max_seq) only
  int Hq, Hkv;
  float sm_scale;
  float* o_part;              // [Hkv][P][G][D]
  float* lse_part;            // [Hkv][P][G]
  int64_t n_partials;
  uint16_t* out;              // [B][Hq][D]
  float* lse_out;             // [B][Hq] or nullptr
};

// Flat mode: the keys of request b (a request longer than max_seq is cut to it, so that its
// partials stay inside its own range) and its partial count.
__device__ __forceinline__ int flat_len(const DecodeArgs& a, int b) { return min(a.seq_lens[b], a.max_seq); }
__device__ __forceinline__ int flat_parts(int len) { return (len + rs::kFlatChunk - 1) / rs::kFlatChunk; }

// One work item per (item, KV head): its key chunk for all query rows of its row tile.
// A request covered by this single item gets its final output here; otherwise the
// item writes one partial (o / l, lse) per (request, head) for decode_merge_kernel.  NT: K/V
// loads with the non-temporal policy.
template <int D, bool NT>
__global__ void __launch_bounds__(kThreads, 2) decode_bf16_kernel(DecodeArgs a) {
  __shared__ Stage<D, kDecKB> sm[kDecNS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int kvh = blockIdx.x % a.Hkv;
  const int item = blockIdx.x / a.Hkv;
  const int row = wave * 32 + (lane & 31);
  const int j = row / G, g = row % G;
  int k0, k1, rep, nreq, b, pidx, nparts;
  if (a.items) {
    const int32_t* it = a.items + item * rs::kItemWords;
    k0 = it[0]; k1 = it[1]; rep = it[2]; nreq = it[3];
    const int4 e = j < nreq ? a.item_req[it[4] + j] : make_int4(rep, 0, 0, 0);
    b = e.x; pidx = e.y; nparts = e.z;
  } else {
    rep = b = item / a.flat_nch;
    const int ch = item % a.flat_nch, len = flat_len(a, b);
    k0 = ch * rs::kFlatChunk;
    k1 = min(k0 + rs::kFlatChunk, len);
    if (k0 >= k1) return;
    nreq = 1; pidx = item; nparts = flat_parts(len);
  }
  const bool valid = j < nreq;
  const int64_t qrow_idx = int64_t(b) * a.Hq + kvh * G + g;
  bf16x8 qf[D / 16];
  load_q<D>(qf, a.q + qrow_idx * D, valid, lane);
  WaveState<D> ws;
  wave_init<D>(ws);
  const bool has_rows = wave * 32 < nreq * G;
  stream_keys<D, kDecKB, kDecNS, true, NT>(ws, sm, qf, a.kpool + int64_t(kvh) * D, a.vpool + int64_t(kvh) * D,
                 a.req_to_token + int64_t(rep) * a.ld, a.Hkv, k0, k1, k1, INT32_MAX,
                 a.sm_scale * kLog2e, has_rows, tid);
  if (!valid) return;
  const float l = ws.l + __shfl_xor(ws.l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = ws.m * a.sm_scale + __logf(l);
  const int hi = lane >> 5;
  if (nparts == 1) {                     // this item covers the request: final output
    uint16_t* orow = a.out + qrow_idx * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = mb * 32 + 8 * q4 + 4 * hi;
        uint2 u;
        u.x = pack_bf16(ws.o[mb][4 * q4 + 0] * inv, ws.o[mb][4 * q4 + 1] * inv);
        u.y = pack_bf16(ws.o[mb][4 * q4 + 2] * inv, ws.o[mb][4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = u;
      }
    if (hi == 0 && a.lse_out) a.lse_out[qrow_idx] = lse;
    return;
  }
  float* orow = a.o_part + ((int64_t(kvh) * a.n_partials + pidx) * G + g) * D;
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = mb * 32 + 8 * q4 + 4 * hi;
      *reinterpret_cast<float4*>(orow + d) =
          make_float4(ws.o[mb][4 * q4 + 0] * inv, ws.o[mb][4 * q4 + 1] * inv, ws.o[mb][4 * q4 + 2] * inv,
                      ws.o[mb][4 * q4 + 3] * inv);
    }
  if (hi == 0) a.lse_part[(int64_t(kvh) * a.n_partials + pidx) * G + g] = lse;
}

// Log-sum-exp merge of each (request, KV head)'s partials:
//   lse = log sum_i exp(lse_i),  o = sum_i exp(lse_i - lse) o_i.
// A second launch: merging inside the decode kernel (the workgroup that writes a request's
// last partial merges it, partials exchanged through agent-scope atomic stores and loads)
// measured 1.6-5x slower, because the last workgroups to finish are the long shared-segment
// items, which then merge dozens of requests one after another.
// A request's partials sit consecutively in the workspace, so the workgroup finds them from
// two numbers.  Each thread owns four consecutive output elements (of one query head) and
// loads the lse and the four values of a batch of kMergeBatch partials at once, so that the
// loads of a batch are in flight together; a running maximum keeps the sums finite across
// batches.
constexpr int kMergeBatch = 16;

template <int D>
__global__ void __launch_bounds__(kThreads) decode_merge_kernel(DecodeArgs a) {
  const int kvh = blockIdx.x % a.Hkv, b = blockIdx.x / a.Hkv;
  int base, n;
  if (a.part_ptr) {
    base = a.part_ptr[b];
    n = a.part_ptr[b + 1] - base;
  } else {
    base = b * a.flat_nch;
    n = flat_parts(flat_len(a, b));
  }
  if (n <= 1) return;
  const int G = a.Hq / a.Hkv;
  const float* op = a.o_part + (int64_t(kvh) * a.n_partials + base) * G * D;   // [n][G][D]
  const float* lp = a.lse_part + (int64_t(kvh) * a.n_partials + base) * G;     // [n][G]
  for (int e0 = 4 * int(threadIdx.x); e0 < G * D; e0 += 4 * kThreads) {
    const int g = e0 / D;
    float m = -INFINITY, sum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i0 = 0; i0 < n; i0 += kMergeBatch) {
      float l[kMergeBatch];
      float4 o[kMergeBatch];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        if (i0 + i < n) {
          l[i] = lp[int64_t(i0 + i) * G + g];
          o[i] = *reinterpret_cast<const float4*>(op + int64_t(i0 + i) * G * D + e0);
        } else {
          l[i] = -INFINITY;
          o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      float mb = m;
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) mb = fmaxf(mb, l[i]);
      // mb is finite: every partial covers at least one key
      const float r = __expf(m - mb);    // 0 before the first batch
      sum *= r;
      acc.x *= r; acc.y *= r; acc.z *= r; acc.w *= r;
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const float w = __expf(l[i] - mb);
        sum += w;
        acc.x = fmaf(w, o[i].x, acc.x);
        acc.y = fmaf(w, o[i].y, acc.y);
        acc.z = fmaf(w, o[i].z, acc.z);
        acc.w = fmaf(w, o[i].w, acc.w);
      }
      m = mb;
    }
    const float inv = 1.f / sum;
    const int64_t orow = int64_t(b) * a.Hq + kvh * G + g;
    uint2 u;
    u.x = pack_bf16(acc.x * inv, acc.y * inv);
    u.y = pack_bf16(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(a.out + orow * D + e0 % D) = u;
    if (a.lse_out && e0 % D == 0) a.lse_out[orow] = m + __logf(sum);
  }
}

// ------------------------------------------------------------------ fp32 extend (matrix cores)
// Extend attention in fp32 on v_mfma_f32_32x32x2_f32 (fp32 products, fp32 sums).  A
// workgroup takes 32 query rows of one request and one KV head -- rows are (token, query
// head of the group) pairs, token-major, as in the bf16 engines -- and its 4 waves split
// the key range in 32-key tiles (wave w takes tiles w, w + 4, ...), each with its own
// softmax state (reference, row sums, O); the four states merge through LDS at the end.
//
// Same operand scheme as the bf16 engines, without LDS staging: each lane loads its own
// operands straight from the pool.
//     S^T = K Q^T:  step s (of D/2) -- lane l gives K[key l%32][dim (D/2)(l/32) + s] as A
//                   and Q[row l%32][same dim] as B, so a lane's K row is D/2 adjacent floats;
//     O^T += V^T P^T: accumulator register j of lane l is key 8(j/4) + 4(l/32) + j%4 for
//                   row l%32, and step j of P V takes exactly those keys: P enters as B
//                   unmoved; block c (of D/32) of the output holds dims (D/32) m + c for
//                   accumulator row m, so a lane's V operands for one key are D/32 adjacent
//                   floats of dims (D/32)(l%32) ...
// A wave loads tile t + 4 (and the slot ids of tile t + 8) before it computes tile t.
//
// Softmax reference: a wave fixes each row's reference at the row's maximum in the first
// tile the wave computes and never moves it (the bf16 engine's first pass takes none;
// here the reference costs no instruction, as below), so the loop
// tracks no maximum and never rescales O (the VALU work of a tile is the exp2 and the row
// sums; measured on gfx950, fp32 MFMAs leave little VALU issue alongside them).  The
// reference enters the scores through the accumulator: the QK chain starts from -ref,
// so its result is already s - ref.  Later weights above 1 are exact in fp32 until
// they near 2^128; a wave whose row sum passes 2^100, or whose O is not finite, makes
// the workgroup find every row's true maximum in a second pass and recompute with it
// (all weights <= 1).
constexpr int kF32Rows = 32;     // query rows per workgroup
constexpr int kF32Waves = 4;
constexpr float kF32SumLimit = 0x1p100f;   // above this a wave's row sum counts as overflowing

template <int D>
struct F32Kv {
  float k[D / 2];          // key l%32, dims [(D/2)(l/32), (D/2)(l/32) + D/2)
  float v[16][D / 32];     // step j: key 8(j/4) + 4(l/32) + j%4, dims (D/32)(l%32) + c
};

// Loads of one tile.  Lane l's key row (its K operand) starts at the byte offset of its slot;
// the V operands of step j come from the row of key 8(j/4) + 4(l/32) + j%4, the same for
// all lanes of a half, so the 32 row offsets go through a per-wave LDS table (one
// broadcast read per step) instead of being recomputed from shuffled slot ids.
template <int D>
__device__ __forceinline__ void f32_kv_load(F32Kv<D>& t, const float* __restrict__ kb, const float* __restrict__ vb,
                                            uint32_t stride, int32_t slot, int lane, uint64_t* vtab) {
  const int h = lane >> 5, n = lane & 31;
  const uint64_t row = uint64_t(uint32_t(slot)) * stride;   // slot ids are non-negative
  const float4* kr = reinterpret_cast<const float4*>(kb + row + (D / 2) * h);
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const float4 x = kr[c];
    t.k[4 * c + 0] = x.x;
    t.k[4 * c + 1] = x.y;
    t.k[4 * c + 2] = x.z;
    t.k[4 * c + 3] = x.w;
  }
  if (h == 0) vtab[n] = row;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float* vr = vb + vtab[8 * (j / 4) + 4 * h + j % 4] + (D / 32) * n;
    if constexpr (D == 64) {
      const float2 x = *reinterpret_cast<const float2*>(vr);
      t.v[j][0] = x.x;
      t.v[j][1] = x.y;
    } else {
      const float4 x = *reinterpret_cast<const float4*>(vr);
      t.v[j][0] = x.x;
      t.v[j][1] = x.y;
      t.v[j][2] = x.z;
      t.v[j][3] = x.w;
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// What one pass over a wave's tiles computes.
enum F32Mode {
  kF32First = 0,   // weights against a reference fixed from the wave's first tile
  kF32Track = 1,   // only each row's maximum score
  kF32Fixed = 2,   // weights against a given reference (the row's true maximum)
};

// One 32-key tile: scores minus the reference (the chain starts from -ref), causal mask
// (keys past the row's position drop out), then by mode: the running maximum, or the
// weights exp2(s - ref) in exp2 units (the scale and log2(e) are folded into the query),
// their row sums and P V.
template <int D, int MODE>
__device__ __forceinline__ void f32_tile(const F32Kv<D>& t, const float (&qv)[D / 2], int key0, int pos,
                                         bool mask, int h, bool& first, f32x16& negref, float& ref, float& lsum,
                                         float& mx, f32x16 (&o)[D / 32]) {
  f32x16 s = __builtin_amdgcn_mfma_f32_32x32x2f32(t.k[0], qv[0], negref, 0, 0, 0);
#pragma unroll
  for (int st = 1; st < D / 2; ++st) s = __builtin_amdgcn_mfma_f32_32x32x2f32(t.k[st], qv[st], s, 0, 0, 0);
  if (mask) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (key0 + 8 * (i / 4) + 4 * h + i % 4 > pos) s[i] = -INFINITY;
  }
  if (MODE == kF32Track) {
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    return;
  }
  if (MODE == kF32First && first) {   // wave-uniform: the wave's first tile sets the reference
    float m = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, s[i]);
    ref = xhalf_max(m);
    const float r = ref == -INFINITY ? 0.f : ref;   // no visible key: none in later tiles either
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] -= r;
      negref[i] = -r;
    }
    first = false;
  }
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s[i] = __builtin_amdgcn_exp2f(s[i]);
    ps += s[i];
  }
  lsum += ps;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int c = 0; c < D / 32; ++c) o[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(t.v[j][c], s[j], o[c], 0, 0, 0);
}

// Per-wave state of one query-row tile and the walk over the wave's key tiles.
struct F32Walk {
  const int32_t* trow;
  const float* kb;
  const float* vb;
  uint32_t stride;
  int nkeys, nkt, pos, pos_min, lane, wave, h, n;
};

template <int D, int NW, int MODE>
__device__ __forceinline__ void f32_pass(const F32Walk& w, const float (&qv)[D / 2], uint64_t* tab, float& ref,
                                         float& lsum, float& mx, f32x16 (&o)[D / 32]) {
  if (w.wave >= w.nkt) return;
  // key indexes past the context repeat its last key: always a real row, weight 0
  auto slot_of = [&](int kt) { return w.trow[min(kt * 32 + w.n, w.nkeys - 1)]; };
  bool first = MODE == kF32First;
  f32x16 negref;
  const float r0 = MODE == kF32Fixed && ref != -INFINITY ? -ref : 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) negref[i] = r0;
  F32Kv<D> ta, tb;
  int kt = w.wave;
  int32_t sa = slot_of(kt);
  f32_kv_load<D>(ta, w.kb, w.vb, w.stride, sa, w.lane, tab);
  int32_t sb = slot_of(kt + NW);
  for (;;) {
    sa = slot_of(kt + 2 * NW);
    f32_kv_load<D>(tb, w.kb, w.vb, w.stride, sb, w.lane, tab);
    f32_tile<D, MODE>(ta, qv, kt * 32, w.pos, kt * 32 + 31 > w.pos_min, w.h, first, negref, ref, lsum, mx, o);
    kt += NW;
    if (kt >= w.nkt) break;
    sb = slot_of(kt + 2 * NW);
    f32_kv_load<D>(ta, w.kb, w.vb, w.stride, sa, w.lane, tab);
    f32_tile<D, MODE>(tb, qv, kt * 32, w.pos, kt * 32 + 31 > w.pos_min, w.h, first, negref, ref, lsum, mx, o);
    kt += NW;
    if (kt >= w.nkt) break;
  }
}

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, 1) extend_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kpool, const float* __restrict__ vpool,
    const int32_t* __restrict__ req_to_token, int64_t ld, const int32_t* __restrict__ qo_indptr,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ extend_lens, int n_qtiles, int Hq, int Hkv,
    float sm_scale, const int32_t* __restrict__ order, float* __restrict__ out) {
  __shared__ float so[NW][D][kF32Rows + 1];   // partial O^T per wave, padded against bank conflicts
  __shared__ float sm[NW][kF32Rows], sl[NW][kF32Rows];
  __shared__ uint64_t vtab[NW][32];            // V row offsets of the tile being loaded, per wave
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = Hq / Hkv;
  const int kvh = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  // requests in the given order; within a request the later (longer) q-tiles first
  const int qt = n_qtiles - 1 - rest % n_qtiles, bi = rest / n_qtiles;
  const int b = order ? order[bi] : bi;
  const int R = extend_lens[b] * G, r0 = qt * kF32Rows;
  if (r0 >= R) return;
  const int prefix = prefix_lens[b], qo = qo_indptr[b];
  const int r_last = min(r0 + kF32Rows, R) - 1;
  F32Walk w;
  w.nkeys = prefix + r_last / G + 1;
  w.nkt = (w.nkeys + 31) / 32;
  w.pos_min = prefix + r0 / G;
  // this lane's query row (rows past the request's end repeat its last row; never stored)
  const int r = min(r0 + n, r_last);
  w.pos = prefix + r / G;
  w.lane = lane;
  w.wave = wave;
  w.h = h;
  w.n = n;
  w.trow = req_to_token + int64_t(b) * ld;
  w.stride = uint32_t(Hkv) * D;
  w.kb = kpool + int64_t(kvh) * D;
  w.vb = vpool + int64_t(kvh) * D;
  const int64_t qoff = (int64_t(qo + r / G) * Hq + kvh * G + r % G) * D;
  const float c = sm_scale * kLog2e;
  float qv[D / 2];
  {
    const float4* qp = reinterpret_cast<const float4*>(q + qoff + (D / 2) * h);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const float4 x = qp[i];
      qv[4 * i + 0] = x.x * c;
      qv[4 * i + 1] = x.y * c;
      qv[4 * i + 2] = x.z * c;
      qv[4 * i + 3] = x.w * c;
    }
  }
  float ref = -INFINITY, lsum = 0.f, mx = -INFINITY;
  f32x16 o[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) o[cb] = f32x16{};
  // O stays in AGPRs through the loop: only MFMAs touch it there
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) asm volatile("" : "+a"(o[cb]));
  f32_pass<D, NW, kF32First>(w, qv, vtab[wave], ref, lsum, mx, o);
  // overflow: a row sum past the limit, or an O that is not finite (x * 0 is NaN exactly
  // for inf and NaN)
  float z = 0.f;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) z = fmaf(o[cb][i], 0.f, z);
  lsum = xhalf_sum(lsum);
  if (__syncthreads_or(!(lsum <= kF32SumLimit) || z != 0.f)) {
    // every row's true maximum over all keys, then the weights again against it
    f32_pass<D, NW, kF32Track>(w, qv, vtab[wave], ref, lsum, mx, o);
    mx = xhalf_max(mx);
    if (h == 0) sm[wave][n] = mx;
    __syncthreads();
    ref = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) ref = fmaxf(ref, sm[v][n]);
    __syncthreads();
    lsum = 0.f;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) o[cb] = f32x16{};
    f32_pass<D, NW, kF32Fixed>(w, qv, vtab[wave], ref, lsum, mx, o);
    lsum = xhalf_sum(lsum);
  }
  // merge the waves' states
  if (h == 0) {
    sm[wave][n] = ref;
    sl[wave][n] = lsum;
  }
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) so[wave][(D / 32) * (8 * (i / 4) + 4 * h + i % 4) + cb][n] = o[cb][i];
  __syncthreads();
  constexpr int kPerThread = D * kF32Rows / (64 * NW);   // output dims per thread
  static_assert(kPerThread % 4 == 0, "float4 stores");
  const int row = tid / (D / kPerThread), d0 = (tid % (D / kPerThread)) * kPerThread;
  if (r0 + row > r_last) return;
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < NW; ++v) M = fmaxf(M, sm[v][row]);
  float e[NW], L = 0.f;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    e[v] = sm[v][row] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[v][row] - M);
    L = fmaf(e[v], sl[v][row], L);
  }
  // each wave's weight share first: e_w / L times a finite O_w cannot overflow
  const float inv = 1.f / L;
#pragma unroll
  for (int v = 0; v < NW; ++v) e[v] *= inv;
  const int rr = r0 + row;
  float* op = out + (int64_t(qo + rr / G) * Hq + kvh * G + rr % G) * D + d0;
#pragma unroll
  for (int i = 0; i < kPerThread; i += 4) {
    float4 x;
    float* xs = reinterpret_cast<float*>(&x);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float acc = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) acc = fmaf(e[v], so[v][d0 + i + k][row], acc);
      xs[k] = acc;
    }
    *reinterpret_cast<float4*>(op + i) = x;
  }
}

// ------------------------------------------------------------------ fp32 decode (VALU)
// One wave per (request, query head): 64 keys per step, a lane per key for the scores,
// the whole wave over the head dims for P V.
template <int D>
__global__ void __launch_bounds__(64) decode_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kpool, const float* __restrict__ vpool,
    const int32_t* __restrict__ req_to_token, int64_t ld, const int32_t* __restrict__ seq_lens, int max_len, int Hq,
    int Hkv, float sm_scale, float* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int DPL = D / 64;                    // output dims per lane
  __shared__ float qs[D];
  const int lane = threadIdx.x;
  const int h = blockIdx.x % Hq, b = blockIdx.x / Hq;
  const int pos = min(seq_lens[b], max_len) - 1;   // a request is cut to max_len keys
  const int G = Hq / Hkv, kvh = h / G;
  const float* qp = q + (int64_t(b) * Hq + h) * D;
  for (int d = lane; d < D; d += 64) qs[d] = qp[d];
  __syncthreads();
  const int32_t* trow = req_to_token + int64_t(b) * ld;
  const int64_t stride = int64_t(Hkv) * D;
  const float* kb = kpool + int64_t(kvh) * D;
  const float* vb = vpool + int64_t(kvh) * D;
  float m = -INFINITY, l = 0.f, o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.f;
  for (int key0 = 0; key0 <= pos; key0 += 64) {
    const int key = key0 + lane;
    const bool ok = key <= pos;
    float s = -INFINITY;
    int64_t slot = 0;
    if (ok) {
      slot = trow[key];
      const float4* kr = reinterpret_cast<const float4*>(kb + slot * stride);
      float acc = 0.f;
#pragma unroll 4
      for (int d4 = 0; d4 < D / 4; ++d4) {
        float4 kv = kr[d4];
        acc = fmaf(qs[4 * d4 + 0], kv.x, acc);
        acc = fmaf(qs[4 * d4 + 1], kv.y, acc);
        acc = fmaf(qs[4 * d4 + 2], kv.z, acc);
        acc = fmaf(qs[4 * d4 + 3], kv.w, acc);
      }
      s = acc * sm_scale;
    }
    float mx = s;
#pragma unroll
    for (int off = 32; off; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float m_new = fmaxf(m, mx);
    const float alpha = __expf(m - m_new);
    const float p = ok ? __expf(s - m_new) : 0.f;
    float ps = p;
#pragma unroll
    for (int off = 32; off; off >>= 1) ps += __shfl_xor(ps, off);
    l = l * alpha + ps;
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] *= alpha;
    const int nvalid = min(64, pos + 1 - key0);
    for (int jj = 0; jj < nvalid; ++jj) {
      const float pj = __shfl(p, jj);
      const int64_t sj = __shfl(slot, jj);
      const float* vr = vb + sj * stride;
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] = fmaf(pj, vr[lane + 64 * k], o[k]);
    }
    m = m_new;
  }
  float* op = out + (int64_t(b) * Hq + h) * D;
#pragma unroll
  for (int k = 0; k < DPL; ++k) op[lane + 64 * k] = o[k] / l;
  if (lse_out && lane == 0) lse_out[int64_t(b) * Hq + h] = m + logf(l);
}

// ------------------------------------------------------------------ small kernels
__global__ void store_kv_kernel(uint4* __restrict__ kpool, uint4* __restrict__ vpool, const uint4* __restrict__ kn,
                                const uint4* __restrict__ vn, const int32_t* __restrict__ slots, int64_t n,
                                int row_chunks) {
  const int64_t total = n * row_chunks;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < total; e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = e / row_chunks, c = e % row_chunks;
    const int64_t dst = int64_t(slots[r]) * row_chunks + c;
    kpool[dst] = kn[e];
    vpool[dst] = vn[e];
  }
}

// Pool rows src[r] -> dst[r], both pools, 16 bytes per thread step.
__global__ void move_kv_kernel(uint4* __restrict__ kpool, uint4* __restrict__ vpool, const int32_t* __restrict__ src,
                               const int32_t* __restrict__ dst, int64_t n, int row_chunks) {
  const int64_t total = n * row_chunks;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < total; e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = e / row_chunks, c = e % row_chunks;
    const int64_t from = int64_t(src[r]) * row_chunks + c, to = int64_t(dst[r]) * row_chunks + c;
    const uint4 k = kpool[from], v = vpool[from];
    kpool[to] = k;
    vpool[to] = v;
  }
}

template <typename T>
__device__ __forceinline__ float ld_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_as_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_as_f32<uint16_t>(const uint16_t* p, int64_t i) { return bf2f(p[i]); }
__device__ __forceinline__ void st_from_f32(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_from_f32(uint16_t* p, int64_t i, float v) { p[i] = f2bf(v); }

template <typename T>
__global__ void merge_states_kernel(const T* __restrict__ oa, const float* __restrict__ la, const T* __restrict__ ob,
                                    const float* __restrict__ lb, int64_t rows, int D, T* __restrict__ o,
                                    float* __restrict__ lse) {
  const int64_t total = rows * D;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < total; e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = e / D;
    const float a = la[r], bb = lb[r];
    const float mx = fmaxf(a, bb);
    const float wa = __expf(a - mx), wb = __expf(bb - mx);
    const float inv = 1.f / (wa + wb);
    st_from_f32(o, e, (wa * ld_as_f32(oa, e) + wb * ld_as_f32(ob, e)) * inv);
    if (lse && e % D == 0) lse[r] = mx + __logf(wa + wb);
  }
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < n; e += int64_t(gridDim.x) * blockDim.x)
    p[e] = 0u;
}

int grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  return int(std::min<int64_t>(std::max<int64_t>(g, 1), 65536));
}

int hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rs::fail(RS_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return RS_OK;
}

bool dims_ok(int32_t Hq, int32_t Hkv, int32_t D) {
  return Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && Hq / Hkv <= rs::kMaxRowsPerItem && (D == 64 || D == 128);
}

// ------------------------------------------------------------------ allocation-free decode scratch
// The workspace of rs_decode_attention_noalloc: a file-scope device array, one per GPU the
// library runs on, held until the process ends.  Host code never uses the array's name as a
// device address (on the host it is only a stand-in for the symbol): the address is looked
// up once per device with hipGetSymbolAddress, with that device current, and kept.
constexpr int64_t kNoallocScratchBytes = int64_t(128) << 20;
__device__ __align__(256) char g_noalloc_scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (nullptr and rs_last_error set on failure).
void* noalloc_scratch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    rs::fail(RS_E_HIP, std::string("rs_decode_attention_noalloc: hipGetDevice: ") + hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    rs::fail(RS_E_UNSUPPORTED, "rs_decode_attention_noalloc: device index beyond " + std::to_string(kMaxDevices));
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_noalloc_scratch));
    if (e != hipSuccess || !p) {
      rs::fail(RS_E_HIP, std::string("rs_decode_attention_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

// ------------------------------------------------------------------ C ABI (device ops)
extern "C" {

int rs_store_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new, const int32_t* slots, int64_t n,
                int32_t Hkv, int32_t D, int32_t dtype, void* stream) {
  if (n < 0 || Hkv <= 0 || D <= 0) return rs::fail(RS_E_INVAL, "rs_store_kv: bad sizes");
  if (n == 0) return RS_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slots) return rs::fail(RS_E_INVAL, "rs_store_kv: null pointer");
  if (dtype != RS_DTYPE_F32 && dtype != RS_DTYPE_BF16) return rs::fail(RS_E_UNSUPPORTED, "rs_store_kv: dtype");
  const int64_t row_bytes = int64_t(Hkv) * D * (dtype == RS_DTYPE_F32 ? 4 : 2);
  if (row_bytes % 16) return rs::fail(RS_E_UNSUPPORTED, "rs_store_kv: a KV row must be a multiple of 16 bytes");
  for (const void* p : {static_cast<const void*>(k_pool), static_cast<const void*>(v_pool), k_new, v_new})
    if (reinterpret_cast<uintptr_t>(p) & 15) return rs::fail(RS_E_INVAL, "rs_store_kv: pointers must be 16-byte aligned");
  const int rc = int(row_bytes / 16);
  hipLaunchKernelGGL(store_kv_kernel, dim3(grid_for(n * rc, 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), static_cast<const uint4*>(k_new),
                     static_cast<const uint4*>(v_new), slots, n, rc);
  return hip_check("rs_store_kv");
}

int rs_move_kv(void* k_pool, void* v_pool, const int32_t* src_slots, const int32_t* dst_slots, int64_t n, int32_t Hkv,
               int32_t D, int32_t dtype, void* stream) {
  if (n < 0 || Hkv <= 0 || D <= 0) return rs::fail(RS_E_INVAL, "rs_move_kv: bad sizes");
  if (dtype != RS_DTYPE_F32 && dtype != RS_DTYPE_BF16) return rs::fail(RS_E_UNSUPPORTED, "rs_move_kv: dtype");
  const int64_t row_bytes = int64_t(Hkv) * D * (dtype == RS_DTYPE_F32 ? 4 : 2);
  if (row_bytes % 16) return rs::fail(RS_E_UNSUPPORTED, "rs_move_kv: a pool row must be a multiple of 16 bytes");
  if (n == 0) return RS_OK;
  if (!k_pool || !v_pool || !src_slots || !dst_slots) return rs::fail(RS_E_INVAL, "rs_move_kv: null pointer");
  if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return rs::fail(RS_E_INVAL, "rs_move_kv: pools must be 16-byte aligned");
  const int rc = int(row_bytes / 16);
  hipLaunchKernelGGL(move_kv_kernel, dim3(grid_for(n * rc, 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), src_slots, dst_slots, n, rc);
  return hip_check("rs_move_kv");
}

int rs_tree_verify_attention(const void* q, const void* k_pool, const void* v_pool, const int32_t* req_to_token,
                             int64_t ld, const int32_t* prefix_lens, const uint64_t* tree_mask, int32_t B, int32_t n,
                             int32_t Hq, int32_t Hkv, int32_t D, float sm_scale, int32_t dtype, void* out,
                             void* stream) {
  if (B < 0 || n < 0 || n > 64 || ld <= 0) return rs::fail(RS_E_INVAL, "rs_tree_verify_attention: bad sizes");
  if (!dims_ok(Hq, Hkv, D)) return rs::fail(RS_E_UNSUPPORTED, "rs_tree_verify_attention: heads/head_dim unsupported");
  if (dtype != RS_DTYPE_BF16) return rs::fail(RS_E_UNSUPPORTED, "rs_tree_verify_attention: bf16 only");
  if (B == 0 || n == 0) return RS_OK;
  if (!q || !k_pool || !v_pool || !req_to_token || !prefix_lens || !tree_mask || !out)
    return rs::fail(RS_E_INVAL, "rs_tree_verify_attention: null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = Hq / Hkv, tpb = kVerifyRows / G;
  const int n_qtiles = (n + tpb - 1) / tpb;
  const int64_t blocks = int64_t(B) * n_qtiles * Hkv;
  if (blocks > INT32_MAX) return rs::fail(RS_E_UNSUPPORTED, "rs_tree_verify_attention: grid too large");
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kThreads), 0, s, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k_pool), static_cast<const uint16_t*>(v_pool), req_to_token, ld,
                       nullptr, prefix_lens, nullptr, n_qtiles, Hq, Hkv, sm_scale, nullptr,
                       static_cast<uint16_t*>(out), int(n), tree_mask, 0);
  };
  if (D == 128) args(extend_bf16_kernel<128, true, 4, 1>);
  else args(extend_bf16_kernel<64, true, 4, 1>);
  return hip_check("rs_tree_verify_attention");
}

int rs_extend_attention(const void* q, const void* k_pool, const void* v_pool, const int32_t* req_to_token,
                        int64_t ld, const int32_t* qo_indptr, const int32_t* prefix_lens, const int32_t* extend_lens,
                        int32_t B, int32_t max_extend_len, int32_t Hq, int32_t Hkv, int32_t D, float sm_scale,
                        int32_t dtype, const int32_t* order, void* out, void* stream) {
  if (B < 0 || max_extend_len < 0 || ld <= 0) return rs::fail(RS_E_INVAL, "rs_extend_attention: bad sizes");
  if (!dims_ok(Hq, Hkv, D)) return rs::fail(RS_E_UNSUPPORTED, "rs_extend_attention: heads/head_dim unsupported");
  if (B == 0 || max_extend_len == 0) return RS_OK;
  if (!q || !k_pool || !v_pool || !req_to_token || !qo_indptr || !prefix_lens || !extend_lens || !out)
    return rs::fail(RS_E_INVAL, "rs_extend_attention: null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == RS_DTYPE_BF16) {
    // 256 query rows per workgroup.  With 4 query heads per KV head and 200-token extends the
    // last q-tile is 87% empty, yet 128-row workgroups (one 32-row block per wave, as the
    // verify kernel) measured 5% slower on that batch: they halve the MFMAs per tile, not
    // the per-tile overhead.
    const int G = Hq / Hkv;
    const int tpb = kExtRows / G;
    const int n_qtiles = (max_extend_len + tpb - 1) / tpb;
    const int64_t blocks = int64_t(B) * n_qtiles * Hkv;
    if (blocks > INT32_MAX) return rs::fail(RS_E_UNSUPPORTED, "rs_extend_attention: grid too large");
    // the longest request's last q-tile takes the one-block loop: start the last tiles last
    // (measured: multi-step agent 0.628 -> 0.596 ms; on the mixed batch, whose q-tiles are all
    // full, deferring them costs 0.8 %, their keys no longer shared in L2)
    const int defer_last = n_qtiles > 1 && (max_extend_len - (n_qtiles - 1) * tpb) * G <= kExtRows / 2;
    auto args = [&](auto kern, int threads) {
      hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(threads), 0, s, static_cast<const uint16_t*>(q),
                         static_cast<const uint16_t*>(k_pool), static_cast<const uint16_t*>(v_pool), req_to_token, ld,
                         qo_indptr, prefix_lens, extend_lens, n_qtiles, Hq, Hkv, sm_scale, order,
                         static_cast<uint16_t*>(out), 0, nullptr, defer_last);
    };
    if (D == 128) args(extend_bf16_kernel<128, false, 4, 2>, 256);
    else args(extend_bf16_kernel<64, false, 4, 2>, 256);
    return hip_check("rs_extend_attention");
  }
  if (dtype == RS_DTYPE_F32) {
    const int64_t rows = int64_t(max_extend_len) * (Hq / Hkv);
    const int64_t n_qtiles = (rows + kF32Rows - 1) / kF32Rows;
    const int64_t blocks = int64_t(B) * n_qtiles * Hkv;
    if (blocks > INT32_MAX) return rs::fail(RS_E_UNSUPPORTED, "rs_extend_attention: grid too large");
    auto kern = D == 128 ? extend_f32_kernel<128, kF32Waves> : extend_f32_kernel<64, kF32Waves>;
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(64 * kF32Waves), 0, s, static_cast<const float*>(q),
                       static_cast<const float*>(k_pool), static_cast<const float*>(v_pool), req_to_token, ld,
                       qo_indptr, prefix_lens, extend_lens, int(n_qtiles), Hq, Hkv, sm_scale, order,
                       static_cast<float*>(out));
    return hip_check("rs_extend_attention");
  }
  return rs::fail(RS_E_UNSUPPORTED, "rs_extend_attention: dtype");
}

int rs_decode_attention(const void* q, const void* k_pool, const void* v_pool, const int32_t* req_to_token, int64_t ld,
                        const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t Hq, int32_t Hkv, int32_t D,
                        float sm_scale, int32_t dtype, const rs_plan* plan, const void* plan_dev, void* ws,
                        int64_t ws_bytes, void* out, float* lse_out, void* stream) {
  if (B < 0 || max_seq_len < 0 || ld <= 0) return rs::fail(RS_E_INVAL, "rs_decode_attention: bad sizes");
  if (ld < max_seq_len) return rs::fail(RS_E_INVAL, "rs_decode_attention: table rows shorter than max_seq_len");
  if (!dims_ok(Hq, Hkv, D)) return rs::fail(RS_E_UNSUPPORTED, "rs_decode_attention: heads/head_dim unsupported");
  if (B == 0) return RS_OK;
  if (!q || !k_pool || !v_pool || !req_to_token || !seq_lens || !out)
    return rs::fail(RS_E_INVAL, "rs_decode_attention: null pointer");
  if (max_seq_len <= 0) return rs::fail(RS_E_INVAL, "rs_decode_attention: every request needs >= 1 key");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == RS_DTYPE_F32) {
    auto kern = D == 128 ? decode_f32_kernel<128> : decode_f32_kernel<64>;
    hipLaunchKernelGGL(kern, dim3(unsigned(int64_t(B) * Hq)), dim3(64), 0, s, static_cast<const float*>(q),
                       static_cast<const float*>(k_pool), static_cast<const float*>(v_pool), req_to_token, ld,
                       seq_lens, max_seq_len, Hq, Hkv, sm_scale, static_cast<float*>(out), lse_out);
    return hip_check("rs_decode_attention");
  }
  if (dtype != RS_DTYPE_BF16) return rs::fail(RS_E_UNSUPPORTED, "rs_decode_attention: dtype");
  if ((plan == nullptr) != (plan_dev == nullptr))
    return rs::fail(RS_E_INVAL, "rs_decode_attention: pass both the plan and its device image, or neither");
  if (reinterpret_cast<uintptr_t>(plan_dev) & 15)
    return rs::fail(RS_E_INVAL, "rs_decode_attention: the plan image must be 16-byte aligned");
  int64_t P, items;
  int flat_nch = 0;
  if (plan) {
    const rs_plan_info_t* pi = rs::plan_info(plan);
    if (pi->B != B || pi->Hq != Hq || pi->Hkv != Hkv || pi->D != D)
      return rs::fail(RS_E_INVAL, "rs_decode_attention: batch or heads differ from the plan's");
    P = pi->n_partials;
    items = pi->n_items;
  } else {
    flat_nch = (max_seq_len + rs::kFlatChunk - 1) / rs::kFlatChunk;
    P = int64_t(B) * flat_nch;
    items = P;
  }
  const rs::WsLayout wl = rs::ws_layout(P, B, Hq, Hkv, D);
  if (!ws || ws_bytes < wl.bytes)
    return rs::fail(RS_E_INVAL, "rs_decode_attention: workspace smaller than rs_decode_workspace_bytes");
  if (items * Hkv > INT32_MAX) return rs::fail(RS_E_UNSUPPORTED, "rs_decode_attention: grid too large");
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kpool = static_cast<const uint16_t*>(k_pool);
  a.vpool = static_cast<const uint16_t*>(v_pool);
  a.req_to_token = req_to_token;
  a.ld = ld;
  a.seq_lens = seq_lens;
  a.items = nullptr;
  a.item_req = nullptr;
  a.part_ptr = nullptr;
  if (plan) {
    const rs::PlanOffsets po = rs::plan_offsets(plan);
    const int32_t* img = static_cast<const int32_t*>(plan_dev);
    a.items = img + po.items;
    a.item_req = reinterpret_cast<const int4*>(img + po.item_req);
    a.part_ptr = img + po.part_ptr;
  }
  a.flat_nch = flat_nch;
  a.max_seq = max_seq_len;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.sm_scale = sm_scale;
  char* w = static_cast<char*>(ws);
  a.o_part = reinterpret_cast<float*>(w + wl.o_off);
  a.lse_part = reinterpret_cast<float*>(w + wl.lse_off);
  a.n_partials = P;
  a.out = static_cast<uint16_t*>(out);
  a.lse_out = lse_out;
  const dim3 g_items(unsigned(items * Hkv)), g_merge(unsigned(int64_t(B) * Hkv));
  // KV bytes the launch streams: the plan's distinct positions, or at most max_seq_len per
  // request in the flat mode
  const int64_t kv_bytes = (plan ? rs::plan_info(plan)->unique_kv_tokens : int64_t(B) * max_seq_len) * Hkv * D * 2 * 2;
  const bool nt = kv_bytes >= kDecodeNtBytes;
  if (D == 128) {
    if (nt) hipLaunchKernelGGL((decode_bf16_kernel<128, true>), g_items, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((decode_bf16_kernel<128, false>), g_items, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(decode_merge_kernel<128>, g_merge, dim3(kThreads), 0, s, a);
  } else {
    if (nt) hipLaunchKernelGGL((decode_bf16_kernel<64, true>), g_items, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((decode_bf16_kernel<64, false>), g_items, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(decode_merge_kernel<64>, g_merge, dim3(kThreads), 0, s, a);
  }
  return hip_check("rs_decode_attention");
}

int rs_decode_attention_noalloc(const void* q, const void* k_pool, const void* v_pool, const int32_t* req_to_token,
                                int64_t ld, const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t Hq,
                                int32_t Hkv, int32_t D, float sm_scale, int32_t dtype, const rs_plan* plan,
                                const void* plan_dev, void* out, float* lse_out, void* stream) {
  int64_t need = 0;
  if (dtype == RS_DTYPE_BF16 && B > 0) {
    need = rs_decode_workspace_bytes(plan, B, max_seq_len, Hq, Hkv, D);
    if (need < 0) return int(need);
    if (need > kNoallocScratchBytes)
      return rs::fail(RS_E_UNSUPPORTED, "rs_decode_attention_noalloc: the batch needs a " + std::to_string(need) +
                                            "-byte workspace, the static scratch holds " +
                                            std::to_string(kNoallocScratchBytes));
  }
  void* ws = need > 0 ? noalloc_scratch() : nullptr;
  if (need > 0 && !ws) return RS_E_HIP;
  return rs_decode_attention(q, k_pool, v_pool, req_to_token, ld, seq_lens, B, max_seq_len, Hq, Hkv, D, sm_scale,
                             dtype, plan, plan_dev, ws, need, out, lse_out, stream);
}

int rs_decode_workspace_init(void* ws, int64_t ws_bytes, void* stream) {
  if (!ws || ws_bytes <= 0 || (ws_bytes & 3) || (reinterpret_cast<uintptr_t>(ws) & 3))
    return rs::fail(RS_E_INVAL, "rs_decode_workspace_init: bad workspace");
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(ws_bytes / 4, 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(ws), ws_bytes / 4);
  return hip_check("rs_decode_workspace_init");
}

int rs_merge_states(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, int64_t rows, int32_t D,
                    int32_t dtype, void* o, float* lse, void* stream) {
  if (rows < 0 || D <= 0) return rs::fail(RS_E_INVAL, "rs_merge_states: bad sizes");
  if (rows == 0) return RS_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o) return rs::fail(RS_E_INVAL, "rs_merge_states: null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = grid_for(rows * D, 256);
  if (dtype == RS_DTYPE_F32)
    hipLaunchKernelGGL(merge_states_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<const float*>(o_a), lse_a,
                       static_cast<const float*>(o_b), lse_b, rows, D, static_cast<float*>(o), lse);
  else if (dtype == RS_DTYPE_BF16)
    hipLaunchKernelGGL(merge_states_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, static_cast<const uint16_t*>(o_a),
                       lse_a, static_cast<const uint16_t*>(o_b), lse_b, rows, D, static_cast<uint16_t*>(o), lse);
  else
    return rs::fail(RS_E_UNSUPPORTED, "rs_merge_states: dtype");
  return hip_check("rs_merge_states");
}

}  // extern "C"
