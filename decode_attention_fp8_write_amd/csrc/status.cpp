// status.cpp — status strings of the C ABI.
#include "pda.h"

extern "C" const char* pda_status_string(int status) {
  switch (status) {
    case PDA_OK: return "ok";
    case PDA_ERR_INVALID_ARG: return "invalid argument";
    case PDA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PDA_ERR_LAUNCH: return "kernel launch failed";
    case PDA_ERR_WORKSPACE: return "workspace too small";
    case PDA_ERR_POOL_EXHAUSTED: return "page pool exhausted";
    case PDA_ERR_SCRATCH:
      return "shape needs more device scratch than paged_decode_attn_noalloc holds";
    default: return "unknown status";
  }
}
