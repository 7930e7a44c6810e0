// Host-side launch interface between the C ABI (sa_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa.h"

// Everything the estimation kernels read, passed by value (theta included).
struct EstArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2;
  int B, Hq, Hkv, G, D, N, bq, bk, sink, local, nQB, nKB;
  int nKT;                 // 64-key tiles of the sequence (the unit keys are staged in)
  float c;                 // softmax scale, fp32
  // workspace carve-out
  int8_t* kq;              // [B, Hkv, nKT * 64, D] int8 keys
  float* sk;               // [B, Hkv, nKB] key-block scales (one per block_k keys)
  int8_t* qq;              // [B, Hkv, nQB, G, D] int8 pooled queries
  float* sq;               // [B, Hkv, nQB, G] pooled-query scales
  float* abar;             // [B, Hkv, nQB, G] block-averaged anchors
  uint32_t* bits;          // [B, Hkv, nQB, W] keep bits
  int8_t* qr;              // relative estimator: int8 query rows [B, Hq, N, D]
  float* sr;               // and their scales [B, Hq, N]
  uint8_t* k4;             // MXFP4 estimator: K codes [B, Hkv, nKT * 64, D / 2]
  uint8_t* k4s;            // and E8M0 scales [B, Hkv, nKT * 64, D / 32]
  int estimator;           // SA_EST_POOLED, SA_EST_RELATIVE or SA_EST_RELATIVE_MXFP4
  int step;                // query blocks per identification group (<= 1: none)
  int W;                   // words per bit row
  // anchor-state reuse (null / 0 otherwise)
  const uint16_t* v;       // values, read by the anchor-state pass
  int64_t vs0, vs1, vs2;
  uint16_t* st_o;          // [B, N, Hq, D] bf16 normalised output over each row's anchor region
  float* st_lse;           // [B, Hq, N] its log-sum-exp (natural log)
  float* xa;               // [B, Hq, N] per-row anchors c * max q.k (workspace)
  int xa_ready;            // 1: the anchor pass reads xa instead of computing it
  // outputs
  int32_t* counts;
  int32_t* idx;
  int32_t stride;
  float* margins;
  float theta[SA_MAX_Q_HEADS];  // per packed head: theta of query head qh[g * G + j]
  // query head of packed head g * G + j (the j-th query head of KV head g): the index of Q, O,
  // LSE and the anchor state in their head dimension
  uint8_t qh[SA_MAX_Q_HEADS];
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
  const int32_t* counts;
  const int32_t* idx;
  int stride;
  int B, Hq, Hkv, G, N, bq, nQB, tpb, n_hp;
  float scale_log2;
  int total;
  // resuming from an anchor state (null otherwise): the sparse pass skips each row's anchor
  // region A(r) = {j <= r : j < sink or j >= r - local + 1} and starts from its output
  const uint16_t* st_o;    // [B, N, Hq, D] bf16
  const float* st_lse;     // [B, Hq, N] natural log
  int sink, local;
  int stripe;              // 1: the lists name key columns (gathered rows), 0: key blocks
  int bk32;                // 1: block lists of 32-key blocks (two per 64-key tile)
  unsigned int* dbg;       // debug builds: the check word (SA_DBG_* bits); unused otherwise
  uint8_t qh[SA_MAX_Q_HEADS];  // query head of packed head g * G + j
};

struct DecArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const uint16_t* ksum;
  const uint8_t* ksum_q4;    // nullable: 4-bit summary codes [B, nKB, Hkv, D/2] (scoring uses these)
  const uint16_t* ksum_scale;  // bf16 scales [B, nKB, Hkv, D/32] of the 4-bit codes
  const uint8_t* ksum_exp;     // nullable: E8M0 exponents [B, nKB, Hkv, D/32] when ksum_q4
                               // holds FP4 (MXFP4) codes instead of the 4-bit integer ones
  const int32_t* cache_len;
  uint16_t* o;
  float* lse;
  int32_t* selected;
  int32_t* sel_count;      // [B, Hkv] blocks selected per (b, g)
  float* scores;           // [B, Hkv, nKBmax]
  float* partial;          // [B, Hq, n_splits, D + 2]
  int64_t qs0, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os2;
  int B, Hq, Hkv, G, D, L, bk, nKB, top_k, sink, local, n_splits;
  float c;
  float top_p;             // 0: fixed K; (0, 1]: top-p budget capped at K
  unsigned int* dbg;       // debug builds: the check word (SA_DBG_* bits); unused otherwise
  uint8_t qh[SA_MAX_Q_HEADS];  // query head of packed head g * G + j
};

hipError_t launch_estimate(const EstArgs& a, int granularity, hipStream_t s);
hipError_t launch_anchor_state(const EstArgs& a, hipStream_t s);
hipError_t launch_prefill(const AttnArgs& a, int D, int granularity, hipStream_t s);
hipError_t launch_block_summary(const DecArgs& a, hipStream_t s);
hipError_t launch_summary_fp4(const uint16_t* ksum, uint8_t* codes, uint8_t* exps, int64_t n_groups,
                              hipStream_t s);
hipError_t launch_summary_q4(const uint16_t* ksum, uint8_t* codes, uint16_t* scales, int64_t n_groups,
                             hipStream_t s);
hipError_t launch_decode(const DecArgs& a, hipStream_t s);
hipError_t launch_head_l1(const uint16_t* o_ref, const uint16_t* o_sp, int B, int N, int Hq, int D,
                          double* err, hipStream_t s);
