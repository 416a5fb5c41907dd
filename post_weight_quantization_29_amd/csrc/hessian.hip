// Calibration Hessian H += 2 X^T X (GPTQ practice page m.lqnn.cn/news/117696,
// section 2.1: the Hessian comes from the layer's input activations).
//
// X is token-major [n_tokens x d], so both MFMA operands have the token index
// as their contraction index and channels contiguous in memory.  Tiles of X
// are copied to LDS exactly as laid out in HBM (channel-contiguous rows) and
// the K-contiguous MFMA operands are produced by the gfx950 transposing LDS
// read ds_read_b64_tr_b16.  Only lower-triangle tiles are computed; the token
// range is split so that enough workgroups exist, each split writes its
// partial tile in the MFMA register order, and a second kernel adds the
// partials in a fixed order into H and mirrors off-diagonal tiles.
#include "common.h"

namespace gptq {

// ---------------------------------------------------------------------------
// tile bookkeeping
// ---------------------------------------------------------------------------
GPTQ_DEV void tri_tile(int q, int& I, int& J) {
  // q enumerates (I, J), I >= J, row by row: q = I(I+1)/2 + J
  int i = (int)((sqrtf(8.0f * (float)q + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= q) ++i;
  while (i * (i + 1) / 2 > q) --i;
  I = i;
  J = q - i * (i + 1) / 2;
}

// Workgroups are dispatched round-robin over the 8 XCDs (XCD = w % 8), each
// with its own L2.  Tiles are ordered by 4x4 super-blocks of the lower
// triangle and cut into 8 contiguous chunks, one per XCD, so the tiles an XCD
// runs share few channel panels; inside an XCD the items run split-major, so
// the co-resident workgroups read the same token range.  Returns false for the
// padding workgroups past the last tile of a chunk.
constexpr int kXCD = 8;
constexpr int kSB = 4;

GPTQ_DEV bool xcd_item(int w, int nt, int ntiles, int splits, int& s, int& I, int& J) {
  const int chunk = (ntiles + kXCD - 1) / kXCD;
  const int x = w % kXCD, k = w / kXCD;
  s = k / chunk;
  const int L = x * chunk + (k - s * chunk);
  if (s >= splits || L >= ntiles) return false;
  // walk the super-blocks (row-major over the lower triangle) to tile number L
  const int nsb = (nt + kSB - 1) / kSB;
  int rem = L;
  for (int ib = 0; ib < nsb; ++ib) {
    const int h = min(kSB, nt - ib * kSB);
    for (int jb = 0; jb <= ib; ++jb) {
      const int wdt = min(kSB, nt - jb * kSB);
      const int cnt = (ib == jb) ? h * (h + 1) / 2 : h * wdt;
      if (rem < cnt) {
        if (ib == jb) {
          int r = 0;
          while (rem >= r + 1) { rem -= r + 1; ++r; }
          I = ib * kSB + r;
          J = jb * kSB + rem;
        } else {
          I = ib * kSB + rem / wdt;
          J = jb * kSB + rem % wdt;
        }
        return true;
      }
      rem -= cnt;
    }
  }
  return false;
}

GPTQ_DEV int tri_index(int I, int J) { return I * (I + 1) / 2 + J; }

// ---------------------------------------------------------------------------
// 16-bit inputs: bf16 / fp16, v_mfma_f32_32x32x16_{bf16,f16}
// Workgroup tile 256x256, 4 waves (2x2) of 128x128, 48 tokens per stage.
//
// Stages are copied HBM -> LDS by buffer_load ... lds (16 bytes per lane, the
// 64 lanes of one instruction fill 1 KB of LDS in lane order) into a ring of
// three slots: stage kk+2 streams in while stage kk is multiplied, so a copy
// has about two stages to land, with no staging registers.  The 16 copies a wave issues per stage are interleaved one per
// MFMA with the first k-slice, so the MFMA pipe keeps running while the
// address unit takes them.  A stage row (one token, 256 channels) is 512 bytes, unpadded;
// its 16-byte chunk c sits at slot c ^ 4*(row % 4), which keeps the
// transposing operand reads free of bank conflicts (the DMA side applies the
// swizzle by permuting the lanes' source addresses).  Tokens past the end and
// channels past d read as zero through the buffer descriptor's range.
// ---------------------------------------------------------------------------
constexpr int kT16 = 256;          // tile edge (channels)
constexpr int kK16 = 32;           // tokens per stage (2 k-slices of 16)
constexpr int kSlots16 = 4;        // LDS ring slots
constexpr int kRow16 = kT16;       // LDS row pitch in elements (512 bytes)
constexpr int kStage16 = kK16 * kRow16;
constexpr int kDiagRows = 4;       // x^2 rows (16-byte chunks) per thread per stage, at most
constexpr int kChunks = kT16 / 8;  // 16-byte chunks per panel row

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// buffer_load_dwordx4 ... lds: each lane's 16 bytes go to LDS at M0 + 16*lane.
// Issued from asm so that the compiler does not model an outstanding LDS write
// (it would otherwise drain every copy in flight before each LDS read); the
// kernel waits for the copies itself with counted s_waitcnt vmcnt.  All
// operands are wave-uniform except the per-lane offset.
GPTQ_DEV void dma16(i32x4_t rsrc, const void* lds_dst, int voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS const void*)lds_dst);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane(rsrc[0]);
  r[1] = __builtin_amdgcn_readfirstlane(rsrc[1]);
  r[2] = __builtin_amdgcn_readfirstlane(rsrc[2]);
  r[3] = __builtin_amdgcn_readfirstlane(rsrc[3]);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(r)
               : "memory", "m0");
}

// workgroup barrier that also stops the compiler from moving memory accesses
// across it, without the fence's drain of outstanding global loads
GPTQ_DEV void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <typename T> struct Op16;
template <> struct Op16<__bf16> {
  typedef bf16x8_t v8;
  typedef bf16x4_t v4;
  static GPTQ_DEV v4 tr(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS v4*)(uintptr_t)addr);
  }
  static GPTQ_DEV f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static GPTQ_DEV float to_f32(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
};
template <> struct Op16<_Float16> {
  typedef f16x8_t v8;
  typedef f16x4_t v4;
  typedef __fp16 raw4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  static GPTQ_DEV v4 tr(uint32_t addr) {
    raw4 r = __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_AS raw4*)(uintptr_t)addr);
    return __builtin_bit_cast(v4, r);
  }
  static GPTQ_DEV f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static GPTQ_DEV float to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
};

// element offset of (token row, channel) inside a stage
GPTQ_DEV int swz16(int row, int ch) { return row * kRow16 + ((((ch >> 3) ^ (4 * (row & 3)))) << 3) + (ch & 7); }

// Transposing read at an LDS byte address (the constant part of the address
// folds into the instruction's offset field).
template <typename T>
GPTQ_DEV typename Op16<T>::v4 tr_at(uint32_t addr) {
  return Op16<T>::tr(addr);
}

// Per-lane byte offset, inside a stage, of the first of a lane's two
// transposing reads for the 32-channel block starting at cbase, k-slice 0.
// The read gives lane j of each 16-lane group g the element (4e + (j%16)/4,
// j%4) of the group's 16x4 block of 64-bit loads; pointing lane 16g+4a+b at
// token 8*(g/2) + a (+4 for the second read) and channels cbase + 16*(g%2) +
// 4b .. +3 hands lane l channel cbase + l%32 at tokens 8*(l/32) + 0..7, i.e.
// MFMA k-slot order.  Token rows of one read differ by multiples of 4, so the
// swizzle term 4*(row%4) = 4a is fixed per lane and k-slice s / second read
// only add 16*s*512 and 4*512 bytes.
GPTQ_DEV uint32_t lane_op_offset(int cbase, int lane) {
  const int g = lane >> 4, a = (lane >> 2) & 3, b = lane & 3;
  const int tok = 8 * (g >> 1) + a;
  const int ch = cbase + 16 * (g & 1) + 4 * b;
  return 2u * (uint32_t)swz16(tok, ch);
}

// s_waitcnt with vmcnt = N (expcnt and lgkmcnt left open)
template <int N>
GPTQ_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
GPTQ_DEV void wait_vm0() { wait_vm<0>(); }

// Every tile also sums x^2 in fp64 for a slice of the channels of its two
// panels (the squares of 16-bit values are exact), in 16-byte chunks of 8
// channels read with one ds_read_b128: tile (I, J) takes slice J of panel I
// and, off the diagonal, slice I of panel J, where slice q of a panel is
// chunks [32q/nt, 32(q+1)/nt).  Each (panel, slice) pair occurs in exactly
// one tile, so every channel is summed once per split, and every tile carries
// a small share of this work.  (Measured: one 16-byte read and 8 squares per
// row in the first waves is faster than spreading 4-channel pieces over all
// four waves.)  These sums are the keys of the
// descending-diagonal column order, so that order does not hinge on fp32
// accumulation rounding.
//
// DIAG = false (no diagonal requested) leaves all of this out.
//
// Partial layout (floats): [work item][wave 4][block 16 = mb*4+nb][reg 16][lane 64]
template <typename T, bool DIAG>
__global__ __launch_bounds__(256, 1) void syrk16_kernel(const T* __restrict__ X, int64_t n_tokens,
                                                         int d, int nt, int ntiles, int splits,
                                                         int nk, float* __restrict__ partial,
                                                         double* __restrict__ pdiag) {
  __shared__ __attribute__((aligned(16))) T sA[kSlots16][kStage16];
  __shared__ __attribute__((aligned(16))) T sB[kSlots16][kStage16];
  constexpr uint32_t kSlotBytes = kStage16 * 2;    // 16 KB
  constexpr uint32_t kSliceBytes = 16 * kRow16 * 2; // 16 token rows
  constexpr int NI = kK16 / 8;                     // copies per panel per lane per stage
  constexpr int NKS = kK16 / 16;                   // k-slices per stage

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t row_bytes = (uint32_t)d * 2u;
  const uint32_t ldsA = (uint32_t)(uintptr_t)(LDS_AS const void*)&sA[0][0];
  const uint32_t ldsB = (uint32_t)(uintptr_t)(LDS_AS const void*)&sB[0][0];

  uint32_t offA[4], offB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    offA[i] = lane_op_offset(wm * 128 + i * 32, lane);
    offB[i] = lane_op_offset(wn * 128 + i * 32, lane);
  }

  // Persistent: workgroup (x = XCD, c) runs items c, c + nper, c + 2*nper, ... of
  // XCD x's list, so the workgroups of an XCD move through the list in rounds
  // and those sharing channel panels read the same tokens at the same time.
  const int x = blockIdx.x % kXCD, c = blockIdx.x / kXCD, nper = gridDim.x / kXCD;
  const int per_xcd = ((ntiles + kXCD - 1) / kXCD) * splits;
  for (int kidx = c; kidx < per_xcd; kidx += nper) {
  int s, I, J;
  if (!xcd_item(kidx * kXCD + x, nt, ntiles, splits, s, I, J)) continue;
  s = __builtin_amdgcn_readfirstlane(s);
  I = __builtin_amdgcn_readfirstlane(I);
  J = __builtin_amdgcn_readfirstlane(J);
  const int w = s * ntiles + tri_index(I, J);     // partial slot
  const int ks0 = __builtin_amdgcn_readfirstlane((int)((int64_t)nk * s / splits));
  const int ks1 = __builtin_amdgcn_readfirstlane((int)((int64_t)nk * (s + 1) / splits));

  // copies of the previous item (and its stores) are complete and every wave
  // is done with its LDS
  wait_vm0();
  lds_barrier();

  // DMA assignment: copy i of wave v fills stage rows R = 8i+2v (lanes 0-31)
  // and 8i+2v+1 (lanes 32-63); lane slot L%32 of row R takes chunk
  // (L%32) ^ 4(R%4), i.e. channels 8*that .. +7 of the panel.  R%4 does not
  // depend on i.
  int voffA[NI], voffB[NI];
  {
    const int R = 2 * wave + (lane >> 5);
    const int cc = (lane & 31) ^ (4 * (R & 3));
    const int chA = I * kT16 + 8 * cc, chB = J * kT16 + 8 * cc;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      voffA[i] = (chA < d) ? (int)((uint32_t)(R + 8 * i) * row_bytes + chA * 2) : 0x7ffffff0;
      voffB[i] = (chB < d) ? (int)((uint32_t)(R + 8 * i) * row_bytes + chB * 2) : 0x7ffffff0;
    }
  }
  // buffer descriptor of stage kk (rows past the end, or kk outside this
  // split, read as zero)
  auto stage_rsrc = [&](int kk) {
    const int64_t t0 = (int64_t)kk * kK16;
    const int64_t rows = (kk < ks1) ? min<int64_t>(kK16, n_tokens - t0) : 0;
    const uint64_t base = reinterpret_cast<uint64_t>(X) + (uint64_t)t0 * row_bytes;
    i32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)(rows * row_bytes));
    r[3] = 0x00020000;
    return r;
  };
  // copy n (0..2*NI-1) of stage kk's DMA into slot `slot`
  auto dma = [&](const i32x4_t& r, int slot, int n) {
    const int i = n % NI;
    const uint32_t dst = ((n < NI) ? ldsA : ldsB) + (uint32_t)slot * kSlotBytes + 4096u * i + 1024u * wave;
    const int voff = (n < NI) ? voffA[i] : voffB[i];
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(voff), "s"(r)
                 : "memory", "m0");
  };

  // fp64 x^2 slices: Cc chunks over P row phases (Cc <= 32, so P >= 8 and a
  // thread takes at most kDiagRows = 4 of a stage's 32 rows)
  const int cA0 = (kChunks * J) / nt, nA = (kChunks * (J + 1)) / nt - cA0;
  const int cB0 = (kChunks * I) / nt, nB = (I != J) ? (kChunks * (I + 1)) / nt - cB0 : 0;
  const int Cc = nA + nB;
  const int P = (Cc > 0) ? kT16 / Cc : 1;
  const int dci = (Cc > 0) ? tid % Cc : 0, dph = (Cc > 0) ? tid / Cc : P;
  const bool dB = dci >= nA;                       // a chunk of panel J (in sB)
  const int dchunk = dB ? cB0 + (dci - nA) : cA0 + dci;
  const int dM = (dph < P) ? (kK16 - dph + P - 1) / P : 0;   // rows dph, dph+P, ... < kK16
  double dsum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) dsum[e] = 0.0;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (ks0 < ks1) {
    // Ring of kSlots16 stage slots.  The sync point of stage k sits before
    // the last k-slice of stage k-1: there every wave has waited for its own
    // copies of stage k (so after the barrier stage k is complete for all) and
    // has finished the earlier slices of stage k-1 (so stage k-2's slot is
    // free and receives stage k + kSlots16 - 2).  The last slice of a stage
    // then overlaps its MFMAs with the reads of the next stage's first slice
    // and with the next copies.
    constexpr int kInFlight = kSlots16 - 3;        // later stages still in flight at a sync point
    static_assert(kSlots16 >= 3 && NKS % 2 == 0, "ring layout");
#pragma unroll
    for (int a = 0; a <= kSlots16 - 3; ++a) {
      const i32x4_t r0 = stage_rsrc(ks0 + a);
#pragma unroll
      for (int n = 0; n < 2 * NI; ++n) dma(r0, a, n);
    }
    wait_vm<kInFlight * 2 * NI>();
    lds_barrier();
    {
      const i32x4_t r0 = stage_rsrc(ks0 + kSlots16 - 2);
#pragma unroll
      for (int n = 0; n < 2 * NI; ++n) dma(r0, kSlots16 - 2, n);
    }
    typename Op16<T>::v4 op[2][8][2];             // [buffer][a0..a3, b0..b3][lo, hi]
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        op[0][f][h] = tr_at<T>((f < 4 ? ldsA + offA[f] : ldsB + offB[f - 4]) + h * 2048u);
    // Stages run in groups of kSlots16 with the ring slot a compile-time
    // constant, so every LDS address is a lane offset plus a constant that
    // folds into the instruction (no per-stage address arithmetic).
    auto stage = [&]<int SLOT>(int kk) {
      constexpr int NSLOT = (SLOT + 1) % kSlots16, DSLOT = (SLOT + kSlots16 - 1) % kSlots16;
      const uint32_t bA = ldsA + (uint32_t)SLOT * kSlotBytes, bB = ldsB + (uint32_t)SLOT * kSlotBytes;
      const uint32_t nA = ldsA + (uint32_t)NSLOT * kSlotBytes, nB = ldsB + (uint32_t)NSLOT * kSlotBytes;
      // this thread's x^2 rows of the stage: one 16-byte chunk each
      const T* dst_ = dB ? sB[SLOT] : sA[SLOT];
      uint4 dv[kDiagRows];
#pragma unroll
      for (int u = 0; u < kDiagRows; ++u)
        if (DIAG && u < dM) dv[u] = *reinterpret_cast<const uint4*>(dst_ + swz16(dph + P * u, 8 * dchunk));
      i32x4_t rn;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        const bool last = (ks == NKS - 1);
        if (last) {
          wait_vm<kInFlight * 2 * NI>();
          lds_barrier();
          rn = stage_rsrc(kk + kSlots16 - 1);
        }
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          const int i = n >> 2, j = n & 3;
          typename Op16<T>::v8 av, bv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            av[e] = op[cur][i][0][e]; av[e + 4] = op[cur][i][1][e];
            bv[e] = op[cur][4 + j][0][e]; bv[e + 4] = op[cur][4 + j][1][e];
          }
          acc[i][j] = Op16<T>::mfma(av, bv, acc[i][j]);
          const int f = n >> 1, h = n & 1;
          if (!last)
            op[nxt][f][h] = tr_at<T>((f < 4 ? bA + offA[f] : bB + offB[f - 4]) +
                                     (uint32_t)(ks + 1) * kSliceBytes + h * 2048u);
          else
            op[nxt][f][h] = tr_at<T>((f < 4 ? nA + offA[f] : nB + offB[f - 4]) + h * 2048u);
          if (last && n < 2 * NI) dma(rn, DSLOT, n);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (DIAG && ks == 0) {
#pragma unroll
          for (int u = 0; u < kDiagRows; ++u) {
            if (u < dM) {
              const uint32_t wv[4] = {dv[u].x, dv[u].y, dv[u].z, dv[u].w};
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint16_t hv = (uint16_t)((e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xFFFFu));
                const double v = (double)Op16<T>::to_f32(hv);
                dsum[e] = fma(v, v, dsum[e]);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    static_assert(kSlots16 == 4, "stage groups of four");
    int kk = ks0;                                  // stage kk uses slot (kk - ks0) % kSlots16
    for (; kk + 4 <= ks1; kk += 4) {
      stage.template operator()<0>(kk);
      stage.template operator()<1>(kk + 1);
      stage.template operator()<2>(kk + 2);
      stage.template operator()<3>(kk + 3);
    }
    if (kk < ks1) stage.template operator()<0>(kk++);
    if (kk < ks1) stage.template operator()<1>(kk++);
    if (kk < ks1) stage.template operator()<2>(kk++);
  }

  float* out = partial + ((size_t)w * 4 + wave) * (16 * 16 * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[((i * 4 + j) * 16 + r) * 64 + lane] = acc[i][j][r];

  // per-phase sums through the first stage slot (copies past the item's end
  // still land in the slots, so wait for them first), added in phase order
  if (!DIAG) continue;
  wait_vm0();
  __syncthreads();
  double* sD = reinterpret_cast<double*>(&sA[0][0]);   // [phase][chunk][8]: P * Cc * 8 <= 2048
  if (dph < P) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sD[(dph * Cc + dci) * 8 + e] = dsum[e];
  }
  __syncthreads();
  if (tid < 8 * Cc) {
    const int ci = tid >> 3, e = tid & 7;
    double t = 0.0;
    for (int ph = 0; ph < P; ++ph) t += sD[(ph * Cc + ci) * 8 + e];
    const bool inB = ci >= nA;
    const int pan = inB ? J : I;
    const int ch = 8 * (inB ? cB0 + (ci - nA) : cA0 + ci) + e;
    pdiag[((size_t)s * nt + pan) * kT16 + ch] = t;
  }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs: v_mfma_f32_32x32x2f32 (lane l supplies A[l%32][k=l/32]).
// Workgroup tile 128x128, 4 waves (2x2) of 64x64, 16 tokens per stage.
// ---------------------------------------------------------------------------
constexpr int kT32 = 128;
constexpr int kK32 = 16;
constexpr int kP32 = kT32 + 32;   // rows 32 banks apart: the two half-waves never collide

__global__ __launch_bounds__(256, 2) void syrk32_kernel(const float* __restrict__ X, int64_t n_tokens,
                                                         int d, int nt, int ntiles, int splits,
                                                         int64_t nk, float* __restrict__ partial,
                                                         double* __restrict__ pdiag) {
  __shared__ __attribute__((aligned(16))) float sA[2][kK32 * kP32];
  __shared__ __attribute__((aligned(16))) float sB[2][kK32 * kP32];
  __shared__ double sD[8][kT32 + 1];
  int s, I, J;
  if (!xcd_item(blockIdx.x, nt, ntiles, splits, s, I, J)) return;
  const int w = s * ntiles + tri_index(I, J);     // partial slot
  const bool diag = (I == J);
  const int64_t ks0 = nk * s / splits, ks1 = nk * (s + 1) / splits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // 16 rows x 128 channels = 512 float4 per panel: 2 per thread
  const int crow = tid >> 5;          // 0..7 (+8)
  const int ccol = (tid & 31) * 4;
  const int chA = I * kT32 + ccol, chB = J * kT32 + ccol;
  const bool okA = chA < d, okB = chB < d;   // d % 8 == 0 => whole float4 in or out
  float4 ra[2], rb[2];
  auto gload = [&](int64_t kstep) {
    const int64_t t0 = kstep * kK32;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t t = t0 + crow + 8 * i;
      const bool tv = t < n_tokens;
      ra[i] = (tv && okA) ? *reinterpret_cast<const float4*>(X + t * d + chA) : make_float4(0, 0, 0, 0);
      if (!diag)
        rb[i] = (tv && okB) ? *reinterpret_cast<const float4*>(X + t * d + chB) : make_float4(0, 0, 0, 0);
    }
  };
  double dsum[4] = {0.0, 0.0, 0.0, 0.0};
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<float4*>(&sA[buf][(crow + 8 * i) * kP32 + ccol]) = ra[i];
      if (!diag) *reinterpret_cast<float4*>(&sB[buf][(crow + 8 * i) * kP32 + ccol]) = rb[i];
    }
    if (diag) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float vv[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) dsum[e] = fma((double)vv[e], (double)vv[e], dsum[e]);
      }
    }
  };
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (ks0 < ks1) {
    gload(ks0);
    lstore(0);
    __syncthreads();
    for (int64_t kk = ks0; kk < ks1; ++kk) {
      const int buf = (int)((kk - ks0) & 1);
      if (kk + 1 < ks1) gload(kk + 1);
      const float* stA = sA[buf];
      const float* stB = diag ? sA[buf] : sB[buf];
#pragma unroll
      for (int k2 = 0; k2 < kK32; k2 += 2) {
        const int row = (k2 + (lane >> 5)) * kP32;
        float a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = stA[row + wm * 64 + i * 32 + (lane & 31)];
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = stB[row + wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      if (kk + 1 < ks1) lstore(buf ^ 1);
      __syncthreads();
    }
  }
  float* out = partial + ((size_t)w * 4 + wave) * (4 * 16 * 64);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[((i * 2 + j) * 16 + r) * 64 + lane] = acc[i][j][r];

  if (diag) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sD[crow][ccol + e] = dsum[e];
    __syncthreads();
    if (tid < kT32) {
      double t = 0.0;
#pragma unroll
      for (int r = 0; r < 8; ++r) t += sD[r][tid];
      pdiag[((size_t)s * nt + I) * kT32 + tid] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// H += 2 * sum_s partial[s]  (fixed order), mirrored for off-diagonal tiles.
// One workgroup per (tile, wave sub-tile); WB = 32-blocks per sub-tile edge.
// ---------------------------------------------------------------------------
template <int WB, int NT>
__global__ __launch_bounds__(NT) void syrk_reduce_kernel(const float* __restrict__ partial,
                                                         float* __restrict__ H, int d, int ntiles,
                                                         int splits) {
  constexpr int E = 32 * WB;            // sub-tile edge
  constexpr int NEL = WB * WB * 1024;   // elements per wave sub-tile
  constexpr int NV = NEL / (4 * NT);    // float4 per thread
  constexpr int TILE = 2 * E;
  __shared__ float sub[E][E + 1];
  const int q = blockIdx.x >> 2, wave = blockIdx.x & 3;
  int I, J;
  tri_tile(q, I, J);
  const int row0 = I * TILE + (wave >> 1) * E;
  const int col0 = J * TILE + (wave & 1) * E;
  const size_t item_stride4 = (size_t)ntiles * 4 * NEL / 4;
  const float4* src = reinterpret_cast<const float4*>(partial + ((size_t)q * 4 + wave) * NEL);
  const int tid = threadIdx.x;
  // the splits are added in fp64 (in a fixed order) and rounded once
  double acc[NV][4];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i][0] = acc[i][1] = acc[i][2] = acc[i][3] = 0.0;
  for (int s = 0; s < splits; ++s) {
    const float4* ps = src + s * item_stride4;
    float4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = ps[tid + NT * i];      // all loads in flight
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      acc[i][0] += v[i].x; acc[i][1] += v[i].y; acc[i][2] += v[i].z; acc[i][3] += v[i].w;
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float a4[4] = {(float)(2.0 * acc[i][0]), (float)(2.0 * acc[i][1]), (float)(2.0 * acc[i][2]),
                         (float)(2.0 * acc[i][3])};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * (tid + NT * i) + u;
      const int blk = e >> 10, r = (e >> 6) & 15, lane = e & 63;
      const int m = (blk / WB) * 32 + mfma32_row(r, lane);
      const int n = (blk % WB) * 32 + mfma32_col(lane);
      sub[m][n] = a4[u];
    }
  }
  __syncthreads();
  // H[row0 + m][col0 + n] += sub[m][n] (rows coalesced), then the mirror
  // H[col0 + n][row0 + m] += sub[m][n]; each batch of 16 reads is issued before
  // its 16 writes so the read-modify-writes do not serialize
  constexpr int NB = 16;
  for (int pass = 0; pass < ((I == J) ? 1 : 2); ++pass) {
    for (int e0 = 0; e0 < E * E; e0 += NT * NB) {
      float old[NB];
      size_t off[NB];
      bool ok[NB];
      float add[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int e = e0 + u * NT + tid;
        const int a = e / E, b = e % E;           // pass 0: (m, n) = (a, b); pass 1: (n, m)
        const int m = pass ? b : a, n = pass ? a : b;
        ok[u] = (e < E * E) && row0 + m < d && col0 + n < d;
        off[u] = pass ? (size_t)(col0 + n) * d + (row0 + m) : (size_t)(row0 + m) * d + (col0 + n);
        add[u] = ok[u] ? sub[m][n] : 0.0f;
        old[u] = ok[u] ? H[off[u]] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (ok[u]) H[off[u]] = old[u] + add[u];
    }
  }
}

// hdiag[c] += 2 * sum_s pdiag[s][c]   (fixed order, fp64)
__global__ __launch_bounds__(256) void diag_reduce_kernel(const double* __restrict__ pdiag, int d,
                                                          int np, int splits,
                                                          double* __restrict__ hdiag) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  double t = 0.0;
  for (int s = 0; s < splits; ++s) t += pdiag[(size_t)s * np + c];
  hdiag[c] += 2.0 * t;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct SyrkPlan {
  int tile;       // 256 (16-bit inputs) or 128 (fp32)
  int ntiles;
  int splits;
  int64_t nk;     // number of token stages
  int nt;         // tile rows
  size_t off_diag;
  size_t ws;      // partial buffers, bytes
};

static SyrkPlan syrk_plan(int64_t n_tokens, int d, bool f32) {
  SyrkPlan p;
  p.tile = f32 ? kT32 : kT16;
  const int kst = f32 ? kK32 : kK16;
  const int nt = (d + p.tile - 1) / p.tile;
  p.nt = nt;
  p.ntiles = nt * (nt + 1) / 2;
  p.nk = (n_tokens + kst - 1) / kst;
  // Pick the split count that minimizes (rounds of 256 resident workgroups per
  // unit of work) plus the partial-sum traffic, with >= 16 stages per split.
  const double tile_flops = 2.0 * p.tile * p.tile * (double)kst;   // per stage
  const double t_stage = tile_flops / (2.5e15 / 256.0 * 0.6);      // s per stage per WG
  const double bytes_tile = (double)p.tile * p.tile * 4.0 * 2.0;    // partial write + read
  double best = 1e300;
  int best_s = 1;
  const int smax = (int)std::max<int64_t>(1, std::min<int64_t>(64, p.nk / 16));
  for (int s = 1; s <= smax; ++s) {
    const double items = (double)kXCD * ((p.ntiles + kXCD - 1) / kXCD) * s;
    const double rounds = std::ceil(items / 256.0);
    const double t = rounds * ((double)p.nk / s) * t_stage + items * bytes_tile / 6.0e12;
    if (t < best * 0.999) { best = t; best_s = s; }
  }
  p.splits = (p.nk == 0) ? 1 : best_s;
  const size_t per_item = (size_t)p.tile * p.tile * sizeof(float);
  p.off_diag = align_up((size_t)p.splits * p.ntiles * per_item);
  p.ws = align_up(p.off_diag + (size_t)p.splits * nt * p.tile * sizeof(double));
  return p;
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_hessian_workspace_size(int64_t n_tokens, int32_t d_in) {
  if (n_tokens < 0 || d_in <= 0) return 0;
  SyrkPlan a = syrk_plan(n_tokens, d_in, false), b = syrk_plan(n_tokens, d_in, true);
  return std::max(a.ws, b.ws);
}

extern "C" int gptq_hessian_accumulate(float* H, double* hdiag, const void* X, gptq_dtype x_dtype,
                                       int64_t n_tokens, int32_t d_in, void* ws, size_t ws_bytes,
                                       hipStream_t s) {
  if (!H || d_in <= 0 || d_in > 65536 || (d_in % 8) != 0 || n_tokens < 0) return GPTQ_ERR_INVALID_ARG;
  if (x_dtype != GPTQ_F32 && x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return GPTQ_OK;
  if (!X) return GPTQ_ERR_INVALID_ARG;
  const bool f32 = (x_dtype == GPTQ_F32);
  SyrkPlan p = syrk_plan(n_tokens, d_in, f32);
  if (!ws || ws_bytes < p.ws || ws_bytes < gptq_hessian_workspace_size(n_tokens, d_in))
    return GPTQ_ERR_WORKSPACE;
  float* partial = static_cast<float*>(ws);
  double* pdiag = reinterpret_cast<double*>(static_cast<char*>(ws) + p.off_diag);
  const unsigned items = (unsigned)(kXCD * ((p.ntiles + kXCD - 1) / kXCD) * p.splits);
  // 16-bit path: one resident workgroup per CU (256 CUs), persistent over items
  const unsigned pgrid = std::min<unsigned>(256u, items);
  const unsigned pg = (pgrid + kXCD - 1) / kXCD * kXCD;
  // the fp64 diagonal only when it is asked for (the 16-bit kernels then do
  // no diagonal work at all; H is the same either way)
  if (x_dtype == GPTQ_BF16) {
    auto k = hdiag ? syrk16_kernel<__bf16, true> : syrk16_kernel<__bf16, false>;
    k<<<pg, 256, 0, s>>>(static_cast<const __bf16*>(X), n_tokens, d_in, p.nt, p.ntiles, p.splits,
                         (int)p.nk, partial, pdiag);
  } else if (x_dtype == GPTQ_F16) {
    auto k = hdiag ? syrk16_kernel<_Float16, true> : syrk16_kernel<_Float16, false>;
    k<<<pg, 256, 0, s>>>(static_cast<const _Float16*>(X), n_tokens, d_in, p.nt, p.ntiles, p.splits,
                         (int)p.nk, partial, pdiag);
  } else {
    syrk32_kernel<<<items, 256, 0, s>>>(static_cast<const float*>(X), n_tokens, d_in, p.nt, p.ntiles,
                                        p.splits, p.nk, partial, pdiag);
  }
  GPTQ_LAUNCH_CHECK();
  if (f32)
    syrk_reduce_kernel<2, 256><<<p.ntiles * 4, 256, 0, s>>>(partial, H, d_in, p.ntiles, p.splits);
  else
    // 512 threads: the 66 KB LDS tile allows two workgroups per CU, so the
    // loads in flight come from more threads per workgroup
    syrk_reduce_kernel<4, 512><<<p.ntiles * 4, 512, 0, s>>>(partial, H, d_in, p.ntiles, p.splits);
  GPTQ_LAUNCH_CHECK();
  if (hdiag) {
    diag_reduce_kernel<<<(d_in + 255) / 256, 256, 0, s>>>(pdiag, d_in, p.nt * p.tile, p.splits, hdiag);
    GPTQ_LAUNCH_CHECK();
  }
  return GPTQ_OK;
}
