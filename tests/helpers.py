"""Shared test plumbing: tensors -> numpy arrays the oracle reads."""
import numpy as np
import torch


def np_of(t):
    """numpy array with the stored bits: bf16 -> uint16 bit patterns, others as is."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def frac(s):
    from fractions import Fraction
    return float(Fraction(s))
