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
    bool raw = false;  // q, k unnormalised; g, beta before -softplus / sigmoid
};

struct PrepArgs {
    const void *q_raw, *k_raw, *g_raw, *b_raw;
    void *q, *k, *g, *beta;
    int64_t T;
    int32_t H, dk;
    bool bf16, head_gate;
};

hipError_t launch_prepare(const PrepArgs& a, hipStream_t stream);

// Carved-up workspace of one kda_chunk_fwd call (all device pointers).
struct ChunkWorkspace {
    WsHeader* header;     // flag + chunk count
    int32_t* cu;          // [N+1] sequence offsets (copied or synthesised)
    int32_t* chunk_off;   // [N+1] first chunk of each sequence
    int2* chunk_tab;      // [max_chunks] first token and length of each chunk
    // Per chunk and head.  "fragment-major": the reduction index is permuted
    // by frag_pos() and every 16 x 32 block is stored as 64 lanes x 8
    // contiguous elements (fm_off()).
    void* W;              // C x dk,  T (beta K exp(b)), fragment-major
    void* QG;             // C x dk,  Q exp(b), fragment-major
    void* KdT;            // dk x C,  (K exp(b_last - b))^T, fragment-major
    void* Up;             // dv x C values of T (beta V): [dv/16][64 lanes][C/4]
    void* P;              // C x C,   masked intra-chunk Q K^T with decay, fragment-major
    float* Gn;            // [max_chunks, H, dk]      exp(b_last)
    // Segmented walk (null when the per-slice walk runs): segments per pair,
    // the start state of every segment after the first, fp32
    // [N*H][G-1][dk][dv], and one published flag per (pair, segment).
    int32_t seg_groups;
    float* seg_state;
    int32_t* seg_flags;   // [N*H][G]
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
    bool raw;  // q, k, g, beta are raw projections (pre-path fused into the intra-chunk kernel)
    int32_t chunk = kChunk;  // tokens per chunk: 64, or 128 (kda_chunk128.hip)
};

// Workspace bytes and carving (host side, shared by size query and launch).
// `chunk` is the chunk size in tokens, 64 or 128.
size_t chunk_workspace_bytes(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16,
                             int32_t chunk = kChunk);
ChunkWorkspace carve_chunk_workspace(void* base, int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv,
                                     bool bf16, int32_t chunk = kChunk);
int64_t max_chunks_for(int64_t T, int32_t N, int32_t chunk = kChunk);
int32_t seg_groups_for(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16, int32_t chunk = kChunk);
bool chunk_grid_fits(int64_t max_chunks, int32_t H, int32_t chunk = kChunk);
// Head sizes and element types the 128-token kernels support (bf16: d_k,
// d_v in {64, 128}; fp32: d_k = d_v = 64, the LDS of one compute unit).
bool chunk128_supported(int32_t dk, int32_t dv, bool bf16);
// The intra-chunk kernel and walk for 128-token chunks, after the chunk map.
hipError_t launch_chunk128_kernels(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream,
                                   hipEvent_t* events);

// Validate cu_seqlens (or synthesise N equal sequences when it is null) and
// write the header, the sequence offsets, the first chunk of every sequence
// and every chunk's first token and length.
// seg_flags: the segmented walk's n_flags flags, cleared with the header
// (null and 0 when it does not run).
hipError_t launch_chunk_map(const int32_t* cu_seqlens, int32_t N, int64_t T, WsHeader* header, int32_t* cu,
                            int32_t* chunk_off, int2* chunk_tab, int32_t* seg_flags, int64_t n_flags,
                            hipStream_t stream, int32_t chunk = kChunk);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Device address, on the current GPU, of the static scratch array of the
// allocation-free chunked forward (KDA_NOALLOC_SCRATCH_BYTES bytes, 256-byte
// aligned); looked up once per device.
hipError_t noalloc_scratch(void** out);
// events: null, or four events recorded before map / intra / walk and after walk.
hipError_t launch_chunk_fwd(const ChunkArgs& a, const ChunkWorkspace& ws, hipStream_t stream,
                            hipEvent_t* events = nullptr);

struct BwdArgs {
    const void *q, *k, *v, *g, *beta;
    const float* S0;            // may be null (zeros)
    const int32_t* cu_seqlens;  // device, may be null
    const void* dO;             // [T, H, dv], element type of q
    const float* dS_T;          // may be null (zeros)
    void *dq, *dk, *dv, *dg, *dbeta;
    float* dS0;                 // may be null (not written)
    int32_t N, H, dk_, dv_;
    int64_t T;
    int64_t max_chunks;
    bool bf16, head_gate;
};

size_t bwd_workspace_bytes(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16);
// The largest number of heads whose intermediates fit in workspace_bytes (0: not even one).
int32_t bwd_head_group(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, bool bf16, size_t workspace_bytes);
hipError_t launch_chunk_bwd(const BwdArgs& a, void* workspace, size_t workspace_bytes, hipStream_t stream);

}  // namespace kda
