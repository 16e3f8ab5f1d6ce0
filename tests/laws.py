"""Expected laws for the driver tests (test-side only)."""
import numpy as np

from tests import synth


def target_law(models) -> np.ndarray:
    """p_t = softmax(z_t / T) in fp64 for every position t of position-only
    models, from the target logits exactly as the library receives them
    (fp32, or bf16 bit patterns): the law every emitted token at position t
    must follow ("Fast Inference from Transformers via Speculative Decoding",
    Appendix A.1)."""
    z = models.target_logits
    z64 = (synth.bf16_bits_to_f32(z) if z.dtype == np.uint16 else z).astype(np.float64) / models.temperature
    z64 = z64 - z64.max(axis=-1, keepdims=True)
    e = np.exp(z64)
    return e / e.sum(axis=-1, keepdims=True)
