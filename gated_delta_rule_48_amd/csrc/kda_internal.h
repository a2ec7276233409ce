// Internal host/device interface between the C ABI (kda_api.hip) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_device.h"

namespace kda {

constexpr int kChunk = 64;  // tokens per chunk (C)

struct DecodeArgs {
    const void *q, *k, *v, *g, *beta;
    float* S;
    void* o;
    int32_t N, H, dk, dv;
    bool bf16, head_gate;
};

// Carved-up workspace of one kda_chunk_fwd call (all device pointers).
struct ChunkWorkspace {
    WsHeader* header;     // flag + chunk count
    int32_t* cu;          // [N+1] sequence offsets (copied or synthesised)
    int32_t* chunk_off;   // [N+1] first chunk of each sequence
    void* W;              // [max_chunks, H, C, dk]   T (beta K exp(b))
    void* QG;             // [max_chunks, H, C, dk]   Q exp(b)
    void* KdT;            // [max_chunks, H, dk, C]   (K exp(b_last - b))^T
    void* Up;             // [max_chunks, H, C, dv]   T (beta V)
    void* P;              // [max_chunks, H, C, C]    masked intra-chunk Q K^T with decay
    float* Gn;            // [max_chunks, H, dk]      exp(b_last)
};

struct ChunkArgs {
    const void *q, *k, *v, *g, *beta;
    const float* S0;
    const int32_t* cu_seqlens;  // device, may be null
    void* o;
    float* S_T;
    int32_t N, H, dk, dv;
    int64_t T;
    int64_t max_chunks;
    bool bf16, head_gate;
};

// Workspace bytes and carving (host side, shared by size query and launch).
size_t chunk_workspace_bytes(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16);
ChunkWorkspace carve_chunk_workspace(void* base, int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv,
                                     bool bf16);
int64_t max_chunks_for(int64_t T, int32_t N);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// events: null, or four events recorded before map / intra / walk and after walk.
hipError_t launch_chunk_fwd(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream,
                            hipEvent_t* events = nullptr);

}  // namespace kda
