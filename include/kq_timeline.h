// Measurement-only extension of the K-quant GEMV library: the per-step timeline
// of a chain.  Exported only by libkq_timeline.so, the build of the same
// sources with -DKQ_TIMELINE (python -m quant_weight_streaming_amd.build
// --timeline); libkq.so has no such symbol and records nothing.
//
// In that build every chain run stores, for each step j and workgroup g of the
// persistent launch, eight 64-bit words at [(j * groups + g) * 8 + k]:
//   k = 0  device clock (s_memrealtime, 100 MHz) when g starts step j
//   k = 1  after g's barrier wait (step j may read step j-1's outputs)
//   k = 2  after g has staged the step's activations in LDS
//   k = 3  after g's main loop (all of its wavefronts)
//   k = 4  after g has written, or handed over, its tiles
//   k = 5  after g's arrival word for step j is stored
// Words 1..4 are written only if g has work in step j (else they keep their
// last value, zero after kq_chain_create).  At j = 0, k = 6 holds the XCC id
// of the workgroup's CU and k = 7 its HW_ID register.  The stamps cost about
// 0.1 us per step; the timeline build is for measurement, not for use.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kq.h"

#ifdef __cplusplus
extern "C" {
#endif

// Copy the stamps of the chain's last completed run to host memory `host`
// (bytes >= n_sub * groups * 64; n_sub counts a mixed-type step once per
// weight type) after a device synchronisation; *groups and *n_sub receive the
// launch's workgroups and sub-steps.  KQ_ERR_SHAPE if `bytes` is too small.
int kq_chain_timeline(kq_chain* c, uint64_t* host, size_t bytes, int* groups, int* n_sub);

#ifdef __cplusplus
}
#endif
