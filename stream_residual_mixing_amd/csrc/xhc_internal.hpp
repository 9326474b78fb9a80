// Host/device shared definitions internal to libxhc (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "xhc.h"

namespace xhc {

constexpr int PT = 64;             // tokens per post block
constexpr int PCH = 4;             // channels per post thread
constexpr int PSLICE = 256 * PCH;  // channels per post block
constexpr int PRE_NKW = 1;         // xHC pre: contraction blocks per wave and stream
constexpr int PRE_WV = 8;          // xHC pre: waves per workgroup
                                   // (a channel slice is PRE_WV x PRE_NKW blocks)

// Everything a call needs, derived once from the config.
struct Plan {
  bool mhc = false;
  int N = 0, K = 0, m = 0, C = 0, B = 0, S = 0, KR = 1;
  long T = 0;
  int dtype = XHC_BF16;
  int iters = 20, use_mgs = 1;
  float eps_norm = 1e-6f, eps_mgs = 1e-6f;
  int ncol_full = 0, ncol_act = 0;  // logical projection widths
  int NTF = 0, NTA = 0;             // 16-column MFMA tiles
  long nkb_full = 0, nkb_act = 0;   // contraction blocks
  int KS = 1;                       // split of the full-state contraction (mHC)
  bool mhc_wide = false;            // mHC: wide maps (N >= 8, bf16) by the 256-token projection kernel
  int nslices = 1;                  // channel slices of the post kernels
  int G = 1;                        // xHC pre: workgroups (channel slices) per 16-token tile
  int Gp = 1;                       // xHC chained: channel slices of the persistent kernels
  long ntiles = 0;                  // xHC pre: 16-token tiles
  // workspace byte offsets
  size_t o_idx = SIZE_MAX, o_p = SIZE_MAX, o_hpre = SIZE_MAX, o_hres = SIZE_MAX, o_hpost = SIZE_MAX,
         o_z = SIZE_MAX, o_gstat = SIZE_MAX, o_wfull = 0, o_wact = SIZE_MAX, o_colsum = SIZE_MAX, o_part = 0, o_stats = 0,
         o_gram = SIZE_MAX, o_part2 = SIZE_MAX, o_sync = SIZE_MAX, o_corr = SIZE_MAX, o_wcoef = SIZE_MAX,
         total = 0;
  // xHC-Flash block (attention + MLP sharing one routing)
  bool flash = false;
  int G2 = 1;                       // splits of the active-row projections
  size_t o_hpre_m = SIZE_MAX, o_hpost_a = SIZE_MAX, o_wact_a = SIZE_MAX;
  size_t o_wq[3] = {SIZE_MAX, SIZE_MAX, SIZE_MAX};   // xHC-Flash-4sub: packed post-maps of sublayers 1-3
};

// xHC pre, fused one-pass kernel.  sync: [0] ticket counter, [1] status
// word, then per tile: arrivals of phase 1, release flag, arrivals of phase 3.
struct XhcPreArgs {
  const void* X;
  void* inp;
  int T, C, m, G, ntiles;
  const uint4* wfull;
  const uint4* wact;
  const float *b_pre, *b_res, *b_post;
  float a_pre, a_res, a_post, eps;
  int iters;
  float* part1;
  float* part2;
  int* sync;
  int* idx;
  float *p, *h_pre, *h_res, *h_post, *z;
  float* gstat;   // per token: the raw pre-map logits [N], then sum x, sum x^2 (for a backward)
};

struct MhcReadArgs {
  const void* X;
  void* inp;
  int T, C, KS;
  const float* part;
  const float* stats;
  const float *b_pre, *b_res, *b_post;
  float a_pre, a_res, a_post;
  int iters;
  float eps;
  float *h_pre, *h_res, *h_post;
};

struct XhcPostArgs {
  void* X;
  const void* out;
  int T, S, C, N, nslices;
  const int* idx;
  const float *p, *h_res, *h_post;
  const float* conv_w;
  int use_mgs;
  float eps_mgs;
  double* gram;   // Gram partials [nslices][T][10]
  // xHC-Flash attention write only: the MLP base readout [T][C] (updated in
  // place) and the MLP pre-map [T][N]
  void* inp_m = nullptr;
  const float* h_pre_m = nullptr;
};

struct MhcPostArgs {
  void* X;
  const void* out;
  int T, C, nslices;
  const float *h_res, *h_post;
};

// Backward workspace layout (xhc_backward.hip).
struct BwdPlan {
  long NC = 0, KC = 0, nkb_f = 0, nkb_a = 0;
  int ncol_f = 0, ncol_a = 0, NTF = 0, NTA = 0, KSa = 1, NBT = 0;
  int nch_f = 1, nch_a = 1, TW_f = 0, TW_a = 0, nch_c = 1, TC = 0;
  size_t o_dhpre = 0, o_dhres = 0, o_dhpost = 0, o_dp = 0, o_xa = 0, o_dxa = 0, o_dg = SIZE_MAX,
         o_cpart = SIZE_MAX,
         o_wpa = 0, o_parta = 0, o_statsa = 0, o_gt = 0, o_ga = 0, o_sc = 0, o_rsel = 0,
         o_brow = 0, o_bsum = 0, o_colsum = 0, o_colpart = 0, o_wpartf = 0, o_wparta = 0, total = 0;
};
bool make_bwd_plan(const Plan& P, BwdPlan* B);
bool launch_xhc_post_backward(const Plan& P, const xhc_weights* w, const void* X, const void* out, const void* d_inp,
                              const void* d_X, void* d_out, float* d_conv, const char* ws, char* bws, hipStream_t st);
bool launch_xhc_pre_backward(const Plan& P, const xhc_weights* w, const void* X, const void* d_inp, const void* d_X,
                             void* dX, const xhc_grads* g, const char* ws, char* bws, hipStream_t st);


bool launch_xhc_pre(const Plan& P, const void* X, void* inp, const xhc_weights* w, char* ws, hipStream_t st);
bool launch_xhc_post(const Plan& P, void* X, const void* out, const xhc_weights* w, char* ws, hipStream_t st);
// The write without allocation: Gram partials in the library's own per-device
// array (post_scratch_bytes of it), whose address noalloc_scratch returns.
size_t post_scratch_bytes(const Plan& P);
hipError_t noalloc_scratch(double** out);
bool launch_xhc_post_noalloc(const Plan& P, void* X, const void* out, const xhc_weights* w, const char* ws,
                             double* scratch_ptr, hipStream_t st);
bool launch_mhc_pre(const Plan& P, const void* X, void* inp, const xhc_weights* w, char* ws, hipStream_t st);
bool launch_mhc_post(const Plan& P, void* X, const void* out, char* ws, hipStream_t st);

// Measurement helper (xhc_probe.hip): a read-only stream of 16-byte loads;
// PROBE_SINK_WORDS workgroups, one word each written to sink.
constexpr unsigned PROBE_SINK_WORDS = 4096;
bool launch_probe_read(const void* src, size_t bytes, uint32_t* sink, int mode, hipStream_t st);

// Weight packing into MFMA B fragments: wf->w_full into wsf (layout Pf),
// wa->w_act into wsa (layout Pa), and the sync words of wsz (layout Pz)
// cleared; each part is skipped when its plan is null.
bool launch_pack(const Plan* Pf, const xhc_weights* wf, char* wsf, const Plan* Pa, const xhc_weights* wa, char* wsa,
                 const Plan* Pz, char* wsz, hipStream_t st);
// Chained xHC sublayers (xhc_chain.hip).
bool launch_xhc_route(const Plan& P, const void* X, const xhc_weights* w, char* ws, hipStream_t st);
bool launch_xhc_pre_chained(const Plan& P, const xhc_weights* w, const Plan* Pn, const xhc_weights* wn,
                            const void* X, void* inp, char* ws, char* wsn, hipStream_t st);
// The rewritten rows' share of the next layer's routing and that layer's
// routing; fuse: also this layer's write (attention-type, chain_post_fused).
bool chain_post_fused(const Plan& P);
bool launch_xhc_chain_tail(const Plan& P, const Plan& Pn, const xhc_weights* w, const xhc_weights* wn, void* X,
                           const void* out, char* ws, char* wsn, bool fuse, hipStream_t st);
// MLP-type write coefficients for the persistent post pass: the Gram pass,
// then per token Q = diag(p) H_post Tm into ws + P.o_wcoef ([T][K][4]).
void launch_xhc_wcoef(const Plan& P, const void* out, const xhc_weights* w, char* ws, hipStream_t st);

// Helpers shared with the xHC-Flash launchers.
void launch_pack_b(int dtype, const void* W, long nkb, int ncol, int NT, void* out, hipStream_t st);
bool launch_projection(int dtype, int NT, const void* X, int T, long K, const void* Wp, long nkb, int KS,
                       float* part, float* stats, hipStream_t st);
bool launch_act_fin(const Plan& P, int G, const float* part2, const float* b_res, const float* b_post, float a_res,
                    float a_post, float* h_res, float* h_post, hipStream_t st);
bool launch_flash_attn_write(const Plan& P, void* X, const void* out, void* inp_m, const char* ws, hipStream_t st);
bool launch_xhc_post_decode(const Plan& P, void* X, const void* out, void* ring, const int* steps,
                            const xhc_weights* w, const char* ws, hipStream_t st);
bool launch_unmixed_write(const Plan& P, int KR, void* X, const void* out, const float* conv_w, char* ws,
                          hipStream_t st);
// xHC-Flash-4sub group (xhc_flash.hip)
bool launch_xhcf4_pre(const Plan& P, const xhcf4_weights* w, const void* X, void* inp, void* bases, char* ws,
                      hipStream_t st);
bool launch_xhcf4_post(const Plan& P, const xhcf4_weights* w, int q, void* X, const void* out, const void* bases,
                       void* inp, char* ws, hipStream_t st);
bool launch_flash_route_p(const Plan& P, const void* X, const void* wp, float* part, const xhcf_weights* w, int* idx,
                          float* p, float* h_pa, float* h_pm, float* z, hipStream_t st);
// xHC-Flash-4sub routing at N = 16 from the LDS-staged persistent projection
// (bf16 state, C a multiple of 128 channels): partials per (16-token tile,
// channel slice) of FLASH4_P1 floats at part, then the routing of every tile.
constexpr size_t FLASH4_P1 = 16 * 80 + 2 * 16 + 16;
struct Flash4Route {
  const float* b_pre[4];
  float a_pre[4];
  int* idx;
  float *p, *z;
  float* h_pre[4];
};
bool flash4_route_p_applies(const Plan& P);
// xHC-Flash readouts at N = 16 staged through LDS (bf16, C a multiple of 128
// channels): npre = 2 (Flash) or 4 with the active streams left out of
// readouts 1.. (Flash-4sub).  False when it does not apply.
bool flash_read_s_applies(const Plan& P);
bool launch_flash_read_s(const Plan& P, const void* X, void* const* out, const float* const* h_pre, const int* idx,
                         int npre, hipStream_t st);
bool launch_flash4_route_p(const Plan& P, const void* X, const void* wp, float* part, const Flash4Route& o,
                           hipStream_t st);
// xHC-Flash block (xhc_flash.hip)
bool launch_xhcf_pre(const Plan& P, const xhcf_weights* w, const void* X, void* inp_a, void* inp_m, char* ws,
                     hipStream_t st);
bool launch_xhcf_mid(const Plan& P, const xhcf_weights* w, void* X, const void* out_a, void* inp_m, char* ws,
                     hipStream_t st);

}  // namespace xhc
