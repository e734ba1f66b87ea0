"""Plain float64 CPU oracle for the Video Delta Attention (VDA) forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) imports, links or calls this package; only the tests, the
``smoke()`` check and the CPU-baseline leg of the benchmark do.  It shares no
code with the GPU path: no kernels, headers, helpers or constants.

Sources (cited by page title and section, never by file position):

* [VDN-summary] "프레임 단위 델타 규칙과 양방향 선형 메모리로 영상 확산 모델의
  어텐션 병목을 걷어낸 Video DeltaNet" (onedev.kr/papers/80).  Sections:
  "어떻게 동작하나" (how it works), "무엇과 다른가" (how it differs),
  "어떻게 쓰나" (how it is used: the token delta rule, the batch form, the
  frame objective, its normal equation and the non-expansion statement),
  "전제와 한계" (premises and limits: inference kernels, anchors excluded
  from the linear state, text counted once).
* [VDN-H3-writeup] "VDN-H3: MiniMax H3 영상을 재생 시간보다 빠르게 생성하는
  하이브리드 어텐션 모델" (discuss.pytorch.kr), section
  "VDN-H3의 하이브리드 어텐션 구조" (the hybrid attention structure).

Every function is pinned by a test in ``tests/test_oracle_*.py`` against
something other than itself (brute-force least squares on the frame
objective, the one-token closed form, library routines, set enumeration,
hand-derived fixtures).  The readings taken where the pages are silent are
listed at the top of ``vda.py``.
"""

from .vda import (  # noqa: F401
    widen_bf16_bits,
    num_chunks,
    anchors,
    window_frames,
    coverage,
    prep,
    frame_stats,
    transition,
    frame_update,
    text_state,
    scan_states,
    query_states,
    readout,
    epilogue,
    forward,
    forward_head,
    token_delta_step,
    batch_form_step,
)
