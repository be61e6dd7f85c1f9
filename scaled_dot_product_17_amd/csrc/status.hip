// Human-readable text of the library's status codes (host only).
#include "attn.h"

extern "C" const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "the sizes must be positive, consistent and fit the library's limits";
        case ATTN_ERR_GQA: return "H_q must be a multiple of H_kv";
        case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (this build supports D = 128)";
        case ATTN_ERR_SCALE: return "scale must be finite";
        case ATTN_ERR_ALIGN: return "bf16 tensors must be 16-byte aligned and fp32 row vectors 4-byte aligned";
        case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
        case ATTN_ERR_LAUNCH: return "kernel launch failed";
        case ATTN_ERR_DEVICE: return "the current device is not a gfx950 GPU";
        case ATTN_ERR_WORKSPACE: return "the workspace is smaller than attn_decode_workspace_bytes()";
        case ATTN_ERR_SCRATCH: return "the call needs more than the library's fixed scratch array (ATTN_DECODE_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}
