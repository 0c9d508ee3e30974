// Internal layout of the KDA forward workspace, shared by the host dispatcher
// and the gfx950 kernels.
//
// The stage-1+2 kernel writes, for every (head h, physical chunk p), one
// fixed-size record that the stage-3+4 kernel streams in chunk order.
// Records are stored chunk-major, record (p, h) at index p * H + h: the
// stage-3+4 workgroups of all heads walk the chunks in step, so at any time
// they read one contiguous region, spread over all HBM channels (a head-major
// order puts the heads a large power-of-two stride apart). The
// record holds the chunk's operands already arranged as MFMA fragments so
// that stage 3+4 loads each fragment with one coalesced 16-byte (bf16) or
// 32-byte (fp32) access per lane:
//
//   W   [rt 0..3][kb 0..K/32-1][lane 0..63][8]   W = A (D_beta K+), rows = chunk position
//   QG  [rt 0..3][kb 0..K/32-1][lane][8]         qg = scale * q * 2^G
//   KG  [rt 0..K/16-1][kb 0..1][lane][8]         kg^T, rows = key channel, k = chunk position
//   AQ  [6][lane][8]                              Aqk (scale folded in, causal mask applied):
//                                                 fragment (rt, kb) for kb <= rt / 2 at index
//                                                 aq_frag(rt, kb); (0, 1) and (1, 1) are all
//                                                 zero and not stored
//   U   [vb 0..V/16-1][rt 0..3][lane][4]         U = A (D_beta V) in accumulator layout
//   GAM [K] float                                 gamma = 2^{G_last} (chunk-end decay)
//
// Fragment element t of lane l (g = l / 16, i = l % 16) holds row i of a
// 16-row tile and the reduction index phys(g, t) of a 32-wide block:
//   phys(g, t) = 4g + t          for t < 4
//              = 16 + 4g + t - 4 for t >= 4
// which is where two stacked 16x16 accumulator tiles keep their rows. This
// lets accumulator tiles feed the next product's B operand without any lane
// shuffle (see kda_device.h).
//
// The metadata region at the start of the workspace serves variable-length
// input (cu_seqlens): per physical chunk its first token and valid length,
// per sequence its first chunk and chunk count, and a longest-first order of
// the sequences, and a small sink that absorbs the output stores of padding
// rows (so that the stores need no branch).
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 64;      // chunk size C of the GPU path
constexpr int kAqFrags = 6;     // stored Aqk fragments per record

// index of Aqk fragment (row tile rt, 32-wide block kb), kb <= rt / 2
__host__ __device__ constexpr int aq_frag(int rt, int kb) { return rt < 2 ? rt : 2 * rt - 2 + kb; }
constexpr int kThreads = 256;   // 4 waves of 64 lanes per workgroup

struct Layout {
  int K, V, elem;               // elem = bytes of the stored element (2 bf16, 4 fp32)
  size_t off_w, off_qg, off_kg, off_aq, off_u, off_gam;  // byte offsets in a record
  size_t rec_bytes;
  size_t ncp;                   // physical chunk slots per head
  int nseq;                     // sequences (varlen) or batch rows (fixed)
  size_t meta_bytes;            // metadata region at the workspace start
  size_t off_chunk_tab, off_seq_tab, off_order;  // byte offsets inside metadata
  size_t off_sink;              // 256-byte target of stores that must be dropped
  size_t total_bytes;
};

static inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// K, V: head dims; elem: 2 or 4; B, T: batch and (packed) length; H: heads;
// nseq: 0 for fixed length, else number of packed sequences.
static inline Layout make_layout(int K, int V, int elem, int64_t B, int64_t T, int64_t H,
                                 int nseq) {
  Layout L{};
  L.K = K;
  L.V = V;
  L.elem = elem;
  const size_t C = kChunk;
  size_t e = (size_t)elem;
  L.off_w = 0;
  L.off_qg = L.off_w + C * K * e;
  L.off_kg = L.off_qg + C * K * e;
  L.off_aq = L.off_kg + C * K * e;
  L.off_u = L.off_aq + (size_t)kAqFrags * 512 * e;
  L.off_gam = L.off_u + C * V * e;
  L.rec_bytes = round_up(L.off_gam + (size_t)K * 4, 256);
  if (nseq > 0) {
    L.ncp = (size_t)((T + kChunk - 1) / kChunk) + (size_t)nseq;
    L.nseq = nseq;
  } else {
    L.ncp = (size_t)B * (size_t)(T / kChunk);
    L.nseq = (int)B;
  }
  L.off_chunk_tab = 64;
  L.off_seq_tab = L.off_chunk_tab + L.ncp * 8;
  L.off_order = L.off_seq_tab + (size_t)L.nseq * 8;
  L.off_sink = round_up(L.off_order + (size_t)L.nseq * 4, 256);
  L.meta_bytes = L.off_sink + 256;
  L.total_bytes = L.meta_bytes + L.rec_bytes * L.ncp * (size_t)H;
  return L;
}

// Backward workspace: the same metadata region as the forward, then one fp32
// slab per (chunk slot p, head h), chunk-major (index p * H + h). Offsets are
// in floats from the slab start; matrices are row-major with the chunk row
// (64) or the key channel (K) first, as named.
struct BwdSlab {
  // chunk terms recomputed from the inputs (natural-log gates; the normalised q,
  // k and the gate cumsum are rebuilt where needed and not stored)
  size_t qg, kg, w, kb;              // [64][K]: s q e^G (bf16 inputs: its transpose [K][64] in bf16,
                                     // first half); k e^(Gl-G); A Kb; beta k e^G
  size_t u, vb;                      // [64][V]: A Vb; beta v (bf16 inputs: W^T [K][64] in bf16, then
                                     // a bf16 copy of kg [64][K])
  size_t aqk, a, m;                  // [64][64]: Aqk (j <= i; fp32 inputs only), (I + L)^-1, M = L / beta (j < i)
  size_t beta, gam, nq, nk;          // [64], [K], [64] row norms of q and k (before the eps clamp)
  // chunk-start state and the gradient of the chunk-end state
  size_t S, dS;                      // [K][V] (bf16, in the first half, for bf16 q/k/v)
  // per-chunk gradients
  size_t dO, vn, dvn, dvb;           // [64][V]
  size_t dqg, dw, dkg, dkb;          // [64][K] (bf16 inputs: dqg holds Aqk^T [64][64] in bf16)
  size_t daqk, da, t1, dl;           // [64][64]
  size_t dgam;                       // [K]
  size_t floats;                     // slab size
};

static inline BwdSlab make_bwd_slab(int K, int V) {
  BwdSlab s{};
  size_t o = 0;
  auto take = [&](size_t n) { const size_t r = o; o += n; return r; };
  const size_t C = kChunk, CK = C * (size_t)K, CV = C * (size_t)V, CC = C * C;
  s.qg = take(CK); s.kg = take(CK); s.w = take(CK); s.kb = take(CK);
  s.u = take(CV); s.vb = take(CV);
  s.aqk = take(CC); s.a = take(CC); s.m = take(CC);
  s.beta = take(C); s.gam = take((size_t)K); s.nq = take(C); s.nk = take(C);
  s.S = take((size_t)K * V); s.dS = take((size_t)K * V);
  s.dO = take(CV); s.vn = take(CV); s.dvn = take(CV); s.dvb = take(CV);
  s.dqg = take(CK); s.dw = take(CK); s.dkg = take(CK); s.dkb = take(CK);
  s.daqk = take(CC); s.da = take(CC); s.t1 = take(CC); s.dl = take(CC);
  s.dgam = take((size_t)K);
  s.floats = round_up(o, 64);
  return s;
}

// total backward workspace bytes (metadata of the forward layout + slabs)
static inline size_t bwd_workspace_bytes(const Layout& L, int64_t H) {
  return L.meta_bytes + L.ncp * (size_t)H * make_bwd_slab(L.K, L.V).floats * sizeof(float);
}

}  // namespace kda
