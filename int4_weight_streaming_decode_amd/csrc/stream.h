// Host-side interface of the streaming decode kernel (stream.hip): one
// persistent launch runs every layer of a batch-1 decode step.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/i4decode.h"

namespace i4d_stream {

// Workspace bytes the kernel needs for a stack of n_layers (layer table, a
// zero block and one exchange region per layer).
size_t region_bytes(const i4d_config* c, int n_layers, int nwg);

// Whether this request can take the streaming kernel: batch 1, int4 weights
// with groups of 128, head_dim 128, every K a multiple of 512, contiguous KV
// caches of one capacity.  Never enqueues anything.
bool supported(const i4d_config* c, int n_layers, const i4d_layer* layers, const i4d_kv* kv, int batch, int nwg);

// Enqueue the step.  region: region_bytes() of workspace (256-byte aligned);
// status: the workspace status word; epoch: a workspace word the kernel
// advances once per launch (zero after i4d_workspace_init).
// timing_ev: null, or two events recorded around the launch.
int run(const i4d_config* c, int n_layers, const i4d_layer* layers, const float* x_in, float* x_out, const i4d_kv* kv,
        const int* pos, int max_pos, char* region, int* status, unsigned* epoch, int nwg, hipStream_t s,
        hipEvent_t* timing_ev);

}  // namespace i4d_stream
